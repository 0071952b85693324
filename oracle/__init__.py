"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the GPU library never does.  It takes the same seeded
cases (``workloads.FiaCase`` / ``workloads.BsaCase``) the GPU path takes and
returns float64 numpy arrays.

Conventions (parity unpinned, a reading of the pages): a row with no allowed
key, and a padding row past the valid length in BNSD/BSND, give out = 0 and
lse = +inf.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_LAYOUT = {"BNSD": 0, "BSND": 1, "BSH": 1, "TND": 2}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Args(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int64), ("QN", ctypes.c_int64), ("KVN", ctypes.c_int64),
        ("Sq", ctypes.c_int64), ("Skv", ctypes.c_int64),
        ("Dqk", ctypes.c_int64), ("Dv", ctypes.c_int64),
        ("lq", ctypes.c_void_p), ("lkv", ctypes.c_void_p),
        ("q_start", ctypes.c_void_p), ("kv_start", ctypes.c_void_p),
        ("scale", ctypes.c_double),
        ("sparse_mode", ctypes.c_int32), ("decode", ctypes.c_int32),
        ("pre_tokens", ctypes.c_int64), ("next_tokens", ctypes.c_int64),
        ("mask", ctypes.c_void_p), ("mask_bstride", ctypes.c_int64),
        ("mask_rstride", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int64),
        ("block_size", ctypes.c_int64), ("pool_layout", ctypes.c_int32),
        ("block_mask", ctypes.c_void_p), ("nqb", ctypes.c_int64), ("nkb", ctypes.c_int64),
        ("X", ctypes.c_int64), ("Y", ctypes.c_int64),
        ("rows", ctypes.c_void_p), ("n_rows", ctypes.c_int64),
        ("kv_i8", ctypes.c_int32), ("kmode", ctypes.c_int32), ("vmode", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("k_off", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p), ("v_off", ctypes.c_void_p),
        ("tok_stride", ctypes.c_int64),
        ("fp8", ctypes.c_int32),
        ("q_bscale", ctypes.c_void_p), ("k_bscale", ctypes.c_void_p), ("v_bscale", ctypes.c_void_p),
        ("nqs", ctypes.c_int64), ("nks", ctypes.c_int64), ("qblk", ctypes.c_int64),
        ("kvblk", ctypes.c_int64),
        ("q_rope", ctypes.c_void_p), ("k_rope", ctypes.c_void_p), ("Dr", ctypes.c_int64),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # FIA_ORACLE_LIB: an already built copy of oracle.c to load instead
        # (the sanitizer check of the pins builds one)
        _lib = ctypes.CDLL(os.environ.get("FIA_ORACLE_LIB") or build())
        _lib.oracle_attention.restype = ctypes.c_int
        _lib.oracle_block_sparse.restype = ctypes.c_int
        _lib.oracle_bsa_compact.restype = ctypes.c_int
        _lib.oracle_read_half.restype = ctypes.c_double
        _lib.oracle_read_half.argtypes = [ctypes.c_uint16, ctypes.c_int]
        _lib.oracle_num_threads.restype = ctypes.c_int
        _lib.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib.oracle_set_threads.restype = None
        _lib.oracle_read_e4m3fn.restype = ctypes.c_double
        _lib.oracle_read_e4m3fn.argtypes = [ctypes.c_uint8]
    return _lib


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's loops over output rows (for timing)."""
    lib().oracle_set_threads(int(n))


def read_half(bits: int, dtype: torch.dtype) -> float:
    return lib().oracle_read_half(bits, 1 if dtype == torch.bfloat16 else 0)


def read_e4m3fn(bits: int) -> float:
    return lib().oracle_read_e4m3fn(bits)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.int8:
        return t.numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    assert t.dtype in (torch.float16, torch.bfloat16), t.dtype
    return t.view(torch.int16).numpy().view(np.uint16)


def _exact_f64(t: torch.Tensor) -> np.ndarray:
    # bf16 / fp32 values widened exactly to double
    return np.ascontiguousarray(t.detach().to("cpu").to(torch.float64).numpy().reshape(-1))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(dtype):
    return 1 if dtype == torch.bfloat16 else 0


def _lengths(case, attr, S):
    L = getattr(case, attr)
    if L is None:
        return np.full(case.B, S, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(L, dtype=np.int64))


def _starts(L):
    return np.ascontiguousarray(np.concatenate([[0], np.cumsum(L)[:-1]]).astype(np.int64))


def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    return r, r.shape[0]


def _outputs(case, rows_n, Dv):
    if rows_n:
        return np.zeros((rows_n, Dv)), np.zeros(rows_n)
    if case.layout == "TND":
        return np.zeros((case.Sq, case.QN, Dv)), np.zeros((case.Sq, case.QN))
    S = 1 if getattr(case, "decode", False) else case.Sq
    if case.layout == "BNSD":
        shape = (case.B, case.QN, S, Dv)
    else:
        shape = (case.B, S, case.QN, Dv)
    return np.zeros(shape), np.zeros((case.B, case.QN, S))


def attention(case, rows=None):
    """Oracle for ``fia``: returns (out, lse) as float64 arrays.  ``out``
    follows the query layout (BSH is returned as BSND) and ``lse`` is
    [B, QN, S] ([T, QN] for TND); with ``rows`` (an iterable of (b, h, i))
    they are [n, Dv] and [n]."""
    keep = []
    a = _Args()
    a.layout = _LAYOUT[case.layout]
    a.dtype = _dtype_code(case.dtype)
    a.B, a.QN, a.KVN = case.B, case.QN, case.KVN
    a.Sq, a.Skv, a.Dqk, a.Dv = case.Sq, case.Skv, case.Dqk, case.Dv
    lq = _lengths(case, "lq", case.Sq)
    lkv = _lengths(case, "lkv", case.Skv)
    keep += [lq, lkv]
    a.lq, a.lkv = _ptr(lq), _ptr(lkv)
    if case.layout == "TND":
        qs, ks = _starts(lq), _starts(lkv)
        keep += [qs, ks]
        a.q_start, a.kv_start = _ptr(qs), _ptr(ks)
    a.scale = float(case.scale)
    a.sparse_mode = int(case.sparse_mode)
    a.decode = 1 if case.decode else 0
    a.pre_tokens, a.next_tokens = int(case.pre_tokens), int(case.next_tokens)
    mla_band = getattr(case, "rope", None) is not None and case.sparse_mode == 4
    if case.atten_mask is not None and case.decode and not mla_band:
        # query S == 1: one value per (batch, kv token), leading 1 broadcasts
        mn = np.ascontiguousarray(case.atten_mask.detach().to("cpu").to(torch.uint8).numpy())
        keep.append(mn)
        a.mask = _ptr(mn)
        a.mask_rstride = 0
        a.mask_bstride = 0 if mn.shape[0] == 1 else mn.shape[-1]
    elif case.atten_mask is not None and case.sparse_mode in (0, 1):
        m = case.atten_mask.detach().to("cpu").contiguous()
        mn = m.to(torch.uint8).numpy()
        keep.append(mn)
        a.mask = _ptr(mn)
        rs = mn.shape[-1]
        a.mask_rstride = rs
        a.mask_bstride = 0 if (mn.ndim == 2 or mn.shape[0] == 1) else mn.shape[-2] * rs
    if case.block_table is not None:
        bt = np.ascontiguousarray(case.block_table.detach().to("cpu").numpy().astype(np.int32))
        keep.append(bt)
        a.block_table = _ptr(bt)
        a.bt_stride = bt.shape[1]
        a.block_size = case.block_size
        a.pool_layout = case.pool_layout
    quant = getattr(case, "quant", None)
    if quant is not None:
        a.kv_i8 = 1
        a.kmode, a.vmode = int(quant["key_quant_mode"]), int(quant["value_quant_mode"])
        for fld, key in (("k_scale", "dequant_scale_key"), ("k_off", "dequant_offset_key"),
                         ("v_scale", "dequant_scale_value"), ("v_off", "dequant_offset_value")):
            t = quant.get(key)
            if t is not None:
                arr = _exact_f64(t)
                keep.append(arr)
                setattr(a, fld, _ptr(arr))
                if (fld[0] == "k" and a.kmode == 1) or (fld[0] == "v" and a.vmode == 1):
                    a.tok_stride = t.shape[-1]
    rope = getattr(case, "rope", None)
    if rope is not None:
        qr, kr = _bits(rope["query_rope"]), _bits(rope["key_rope"])
        keep += [qr, kr]
        qd = int(rope["query_rope"].shape[-1])
        a.q_rope, a.k_rope = _ptr(qr), _ptr(kr)
        a.Dr = qd // case.QN if case.layout == "BSH" else qd     # BSH: H = N * Dr
    r, n = _rows_arg(rows)
    if r is not None:
        keep.append(r)
        a.rows, a.n_rows = _ptr(r), n
    q, k, v = _bits(case.q), _bits(case.k), _bits(case.v)
    out, lse = _outputs(case, n, case.Dv)
    rc = lib().oracle_attention(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    return out, lse


def block_sparse(case, rows=None):
    """Oracle for ``bsa``: (out, lse) as in :func:`attention`."""
    keep = []
    a = _Args()
    a.layout = _LAYOUT[case.layout]
    a.dtype = _dtype_code(case.dtype)
    a.B, a.QN, a.KVN = case.B, case.QN, case.KVN
    a.Sq, a.Skv, a.Dqk, a.Dv = case.Sq, case.Skv, case.D, case.D
    lq = _lengths(case, "lq", case.Sq)
    lkv = _lengths(case, "lkv", case.Skv)
    keep += [lq, lkv]
    a.lq, a.lkv = _ptr(lq), _ptr(lkv)
    if case.layout == "TND":
        qs, ks = _starts(lq), _starts(lkv)
        keep += [qs, ks]
        a.q_start, a.kv_start = _ptr(qs), _ptr(ks)
    a.scale = float(case.scale)
    bm = np.ascontiguousarray(case.block_mask.detach().to("cpu").to(torch.uint8).numpy())
    keep.append(bm)
    a.block_mask = _ptr(bm)
    a.nqb, a.nkb = bm.shape[2], bm.shape[3]
    a.X, a.Y = case.X, case.Y
    fp8 = getattr(case, "fp8", None)
    if fp8 is not None:
        a.fp8 = 1
        for fld, key in (("q_bscale", "dequant_scale_query"), ("k_bscale", "dequant_scale_key"),
                         ("v_bscale", "dequant_scale_value")):
            arr = _exact_f64(fp8[key])
            keep.append(arr)
            setattr(a, fld, _ptr(arr))
        a.nqs, a.nks = fp8["dequant_scale_query"].shape[2], fp8["dequant_scale_key"].shape[2]
        a.qblk, a.kvblk = case.X, case.Y
    r, n = _rows_arg(rows)
    if r is not None:
        keep.append(r)
        a.rows, a.n_rows = _ptr(r), n
    q, k, v = _bits(case.q), _bits(case.k), _bits(case.v)
    out, lse = _outputs(case, n, case.D)
    rc = lib().oracle_block_sparse(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse))
    if rc != 0:
        raise RuntimeError(f"oracle_block_sparse failed ({rc})")
    return out, lse


def bsa_compact(block_mask, lq, lkv, X, Y):
    """Compacted schedule: (idx int32 [B,N,nqb,nkb] ascending with -1 tail,
    cnt int32 [B,N,nqb])."""
    bm = np.ascontiguousarray(np.asarray(block_mask, dtype=np.uint8))
    B, N, nqb, nkb = bm.shape
    lq = np.ascontiguousarray(np.asarray(lq, dtype=np.int64))
    lkv = np.ascontiguousarray(np.asarray(lkv, dtype=np.int64))
    idx = np.zeros((B, N, nqb, nkb), dtype=np.int32)
    cnt = np.zeros((B, N, nqb), dtype=np.int32)
    lib().oracle_bsa_compact(_ptr(bm), ctypes.c_int64(B), ctypes.c_int64(N), ctypes.c_int64(nqb),
                             ctypes.c_int64(nkb), _ptr(lq), _ptr(lkv), ctypes.c_int64(X),
                             ctypes.c_int64(Y), _ptr(idx), _ptr(cnt))
    return idx, cnt
