"""ctypes mirror of include/fia.h: the same entry points under the same names,
argument marshalling only.  Every step of the computation runs in libfia.so;
there is no fallback: if the library is missing, loading raises."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfia.so")

# fia_status
FIA_OK = 0
FIA_ERR_NULLPTR = 1
FIA_ERR_DTYPE = 2
FIA_ERR_SHAPE = 3
FIA_ERR_LAYOUT = 4
FIA_ERR_PARAM = 5
FIA_ERR_UNSUPPORTED = 6
FIA_ERR_WORKSPACE = 7
FIA_ERR_HIP = 8

# fia_dtype
FIA_F16, FIA_BF16, FIA_F32, FIA_I8, FIA_U8, FIA_BOOL, FIA_I32, FIA_I64, FIA_F8E4M3 = range(9)


class fia_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("dims", ctypes.c_int64 * 8)]


class fia_params(ctypes.Structure):
    _fields_ = [
        ("input_layout", ctypes.c_char_p),
        ("num_heads", ctypes.c_int64),
        ("num_key_value_heads", ctypes.c_int64),
        ("scale_value", ctypes.c_double),
        ("pre_tokens", ctypes.c_int64),
        ("next_tokens", ctypes.c_int64),
        ("sparse_mode", ctypes.c_int64),
        ("block_size", ctypes.c_int64),
        ("inner_precise", ctypes.c_int64),
        ("return_softmax_lse", ctypes.c_int32),
        ("actual_seq_qlen", ctypes.c_void_p),
        ("n_actual_seq_qlen", ctypes.c_int64),
        ("actual_seq_kvlen", ctypes.c_void_p),
        ("n_actual_seq_kvlen", ctypes.c_int64),
        ("dequant_scale_key", ctypes.POINTER(fia_tensor)),
        ("dequant_scale_value", ctypes.POINTER(fia_tensor)),
        ("dequant_offset_key", ctypes.POINTER(fia_tensor)),
        ("dequant_offset_value", ctypes.POINTER(fia_tensor)),
        ("key_quant_mode", ctypes.c_int64),
        ("value_quant_mode", ctypes.c_int64),
        ("query_rope", ctypes.POINTER(fia_tensor)),
        ("key_rope", ctypes.POINTER(fia_tensor)),
    ]


class bsa_params(ctypes.Structure):
    _fields_ = [
        ("q_input_layout", ctypes.c_char_p),
        ("kv_input_layout", ctypes.c_char_p),
        ("num_heads", ctypes.c_int64),
        ("num_key_value_heads", ctypes.c_int64),
        ("scale_value", ctypes.c_double),
        ("block_shape", ctypes.c_int64 * 2),
        ("actual_seq_lengths", ctypes.c_void_p),
        ("n_actual_seq_lengths", ctypes.c_int64),
        ("actual_seq_lengths_kv", ctypes.c_void_p),
        ("n_actual_seq_lengths_kv", ctypes.c_int64),
        ("mask_type", ctypes.c_int64),
        ("block_size", ctypes.c_int64),
        ("inner_precise", ctypes.c_int64),
        ("pre_tokens", ctypes.c_int64),
        ("next_tokens", ctypes.c_int64),
        ("softmax_lse_flag", ctypes.c_int32),
        ("dequant_scale_query", ctypes.POINTER(fia_tensor)),
        ("dequant_scale_key", ctypes.POINTER(fia_tensor)),
        ("dequant_scale_value", ctypes.POINTER(fia_tensor)),
    ]


_T = ctypes.POINTER(fia_tensor)
_SIGS = {
    "fia_params_init": (None, [ctypes.POINTER(fia_params)]),
    "bsa_params_init": (None, [ctypes.POINTER(bsa_params)]),
    "fia_get_workspace_size": (ctypes.c_int, [_T, _T, _T, _T, _T, ctypes.POINTER(fia_params), _T, _T,
                                              ctypes.POINTER(ctypes.c_uint64),
                                              ctypes.POINTER(ctypes.c_void_p)]),
    "fia_run": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]),
    "bsa_get_workspace_size": (ctypes.c_int, [_T, _T, _T, _T, _T, _T, ctypes.POINTER(bsa_params), _T,
                                              _T, ctypes.POINTER(ctypes.c_uint64),
                                              ctypes.POINTER(ctypes.c_void_p)]),
    "bsa_run": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]),
    "bsa_schedule_layout": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64),
                                           ctypes.POINTER(ctypes.c_uint64),
                                           ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(ctypes.c_int64)]),
    "fia_run_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "fia_plan_destroy": (None, [ctypes.c_void_p]),
    "fia_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libfia.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  -- loads the HIP runtime the library binds to
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run attention_fia_fwd_amd.build.build() "
                               "(there is no fallback path)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


# Same names as the C ABI -----------------------------------------------------

def fia_params_init(p: fia_params) -> None:
    lib().fia_params_init(ctypes.byref(p))


def bsa_params_init(p: bsa_params) -> None:
    lib().bsa_params_init(ctypes.byref(p))


def _tp(t):
    return ctypes.byref(t) if t is not None else None


def fia_get_workspace_size(query, key, value, atten_mask, block_table, params, attention_out,
                           softmax_lse):
    """Returns (status, workspace_size, plan_handle)."""
    ws = ctypes.c_uint64(0)
    plan = ctypes.c_void_p(None)
    st = lib().fia_get_workspace_size(_tp(query), _tp(key), _tp(value), _tp(atten_mask),
                                      _tp(block_table), ctypes.byref(params), _tp(attention_out),
                                      _tp(softmax_lse), ctypes.byref(ws), ctypes.byref(plan))
    return st, ws.value, plan.value


def fia_run(workspace: int, workspace_size: int, plan: int, stream: int) -> int:
    return lib().fia_run(workspace or None, workspace_size, plan, stream or None)


def bsa_get_workspace_size(query, key, value, block_sparse_mask, atten_mask, block_table, params,
                           attention_out, softmax_lse):
    ws = ctypes.c_uint64(0)
    plan = ctypes.c_void_p(None)
    st = lib().bsa_get_workspace_size(_tp(query), _tp(key), _tp(value), _tp(block_sparse_mask),
                                      _tp(atten_mask), _tp(block_table), ctypes.byref(params),
                                      _tp(attention_out), _tp(softmax_lse), ctypes.byref(ws),
                                      ctypes.byref(plan))
    return st, ws.value, plan.value


def bsa_run(workspace: int, workspace_size: int, plan: int, stream: int) -> int:
    return lib().bsa_run(workspace or None, workspace_size, plan, stream or None)


FIA_NOALLOC_MAX_WORKSPACE = 32 << 20


def fia_run_noalloc(plan: int, stream: int) -> int:
    return lib().fia_run_noalloc(plan, stream or None)


def bsa_schedule_layout(plan: int):
    c, i = ctypes.c_uint64(0), ctypes.c_uint64(0)
    nq, nk = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib().bsa_schedule_layout(plan, ctypes.byref(c), ctypes.byref(i), ctypes.byref(nq),
                                   ctypes.byref(nk))
    return st, c.value, i.value, nq.value, nk.value


def fia_plan_destroy(plan: int) -> None:
    if plan:
        lib().fia_plan_destroy(plan)


def fia_status_string(status: int) -> str:
    return lib().fia_status_string(status).decode()
