"""MI355X (gfx950) fused inference attention forward.

Torch-facing front end of libfia.so.  PyTorch supplies device memory (inputs,
outputs, workspace) and the current HIP stream; every step of the attention
runs in the library's HIP kernels.  The two-phase C ABI (include/fia.h) is
re-exported under its own names from ``attention_fia_fwd_amd._abi``.

    out, lse = fused_infer_attention_score(q, k, v, num_heads=..., input_layout=...,
                                           sparse_mode=3, softmax_scale=...,
                                           return_softmax_lse=True)
    out, lse = block_sparse_attention(q, k, v, block_sparse_mask, num_heads=...)

Argument names and defaults follow the parameter description of
"torch_npu.npu_fused_infer_attention_score_v2" and the constraints of
"aclnnBlockSparseAttentionV2".
"""
from __future__ import annotations

import ctypes
import time
from typing import Optional, Sequence

import numpy as np
import torch

from . import _abi
from ._abi import (FIA_OK, bsa_get_workspace_size, bsa_params, bsa_params_init, bsa_run,
                   bsa_schedule_layout, fia_get_workspace_size, fia_params, fia_params_init,
                   fia_plan_destroy, fia_run, fia_run_noalloc, fia_status_string, fia_tensor)

INT_MAX = 2147483647

_DTYPES = {
    torch.float16: _abi.FIA_F16, torch.bfloat16: _abi.FIA_BF16, torch.float32: _abi.FIA_F32,
    torch.int8: _abi.FIA_I8, torch.uint8: _abi.FIA_U8, torch.bool: _abi.FIA_BOOL,
    torch.int32: _abi.FIA_I32, torch.int64: _abi.FIA_I64,
    torch.float8_e4m3fn: _abi.FIA_F8E4M3,
}


class FiaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fia_status_string(status)}")
        self.status = status


def build() -> str:
    from .build import build as _build
    return _build()


def describe(t: Optional[torch.Tensor]) -> Optional[fia_tensor]:
    """fia_tensor for a dense torch tensor (None stays None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("non-contiguous tensors are not supported")
    d = fia_tensor()
    d.data = t.data_ptr() if t.numel() else 0
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i, s in enumerate(t.shape):
        d.dims[i] = s
    return d


def _host_i64(x):
    if x is None:
        return None, 0, None
    a = np.ascontiguousarray(np.asarray(list(x) if not isinstance(x, np.ndarray) else x,
                                        dtype=np.int64).reshape(-1))
    return a.ctypes.data_as(ctypes.c_void_p), a.size, a


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class FiaPlan:
    """A phase-1 plan plus its workspace and outputs; ``run()`` is phase 2 on
    the current stream.  Reuse it to run the same call repeatedly."""

    def __init__(self, query, key, value, *, atten_mask=None, block_table=None,
                 actual_seq_qlen: Optional[Sequence[int]] = None,
                 actual_seq_kvlen: Optional[Sequence[int]] = None, num_heads: int = 1,
                 num_key_value_heads: int = 0, softmax_scale: float = 1.0,
                 pre_tokens: int = INT_MAX, next_tokens: int = INT_MAX,
                 input_layout: str = "BSH", sparse_mode: int = 0, block_size: int = 0,
                 inner_precise: int = 0, return_softmax_lse: bool = False,
                 dequant_scale_key=None, dequant_scale_value=None, dequant_offset_key=None,
                 dequant_offset_value=None, key_quant_mode: int = 0, value_quant_mode: int = 0,
                 query_rope=None, key_rope=None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
        self.plan = None
        kvn = num_key_value_heads or num_heads
        if block_table is not None:
            Dv = value.shape[-1] if value.dim() == 4 else value.shape[-1] // kvn
        elif input_layout == "BSH":
            Dv = value.shape[-1] // kvn
        else:
            Dv = value.shape[-1]
        if out is None:
            if input_layout == "BSH":
                shape = (*query.shape[:-1], num_heads * Dv)
            else:
                shape = (*query.shape[:-1], Dv)
            out = torch.empty(shape, dtype=query.dtype, device=query.device)
        if return_softmax_lse and lse is None:
            if input_layout == "TND":
                lse = torch.empty(query.shape[0], num_heads, 1, dtype=torch.float32,
                                  device=query.device)
            else:
                S = query.shape[2] if input_layout == "BNSD" else query.shape[1]
                lse = torch.empty(query.shape[0], num_heads, S, 1, dtype=torch.float32,
                                  device=query.device)
        self.out, self.lse = out, (lse if return_softmax_lse else None)
        quant = (dequant_scale_key, dequant_scale_value, dequant_offset_key, dequant_offset_value)
        self._keep = (query, key, value, atten_mask, block_table, out, lse, query_rope, key_rope) + quant
        p = fia_params()
        fia_params_init(p)
        self._layout = input_layout.encode()
        p.input_layout = self._layout
        p.num_heads = num_heads
        p.num_key_value_heads = num_key_value_heads
        p.scale_value = softmax_scale
        p.pre_tokens, p.next_tokens = pre_tokens, next_tokens
        p.sparse_mode = sparse_mode
        p.block_size = block_size
        p.inner_precise = inner_precise
        p.return_softmax_lse = 1 if return_softmax_lse else 0
        qp, qn, qa = _host_i64(actual_seq_qlen)
        kp, kn, ka = _host_i64(actual_seq_kvlen)
        p.actual_seq_qlen, p.n_actual_seq_qlen = qp, qn
        p.actual_seq_kvlen, p.n_actual_seq_kvlen = kp, kn
        self._qdesc = [describe(t) for t in quant]
        (p.dequant_scale_key, p.dequant_scale_value, p.dequant_offset_key,
         p.dequant_offset_value) = [ctypes.pointer(d) if d is not None else None for d in self._qdesc]
        p.key_quant_mode, p.value_quant_mode = key_quant_mode, value_quant_mode
        self._rdesc = [describe(t) for t in (query_rope, key_rope)]
        p.query_rope, p.key_rope = [ctypes.pointer(d) if d is not None else None for d in self._rdesc]
        args = (describe(query), describe(key), describe(value), describe(atten_mask),
                describe(block_table), p, describe(out),
                describe(lse) if return_softmax_lse else None)
        t0 = time.perf_counter()
        st, ws, plan = fia_get_workspace_size(*args)
        self.phase1_s = time.perf_counter() - t0     # the C call alone (validation, plan, upload)
        del qa, ka
        if st != FIA_OK:
            raise FiaError(st, "fia_get_workspace_size")
        self.plan = plan
        self.workspace_size = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
        self.device = query.device

    def run(self):
        st = fia_run(self.workspace.data_ptr(), self.workspace_size, self.plan,
                     _stream_handle(self.device))
        if st != FIA_OK:
            raise FiaError(st, "fia_run")
        return self.out, self.lse

    def run_noalloc(self):
        """Phase 2 on the library's static device scratch (fia_run_noalloc)."""
        st = fia_run_noalloc(self.plan, _stream_handle(self.device))
        if st != FIA_OK:
            raise FiaError(st, "fia_run_noalloc")
        return self.out, self.lse

    def close(self):
        if self.plan:
            fia_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class BsaPlan:
    """Phase-1 plan of block-sparse attention with workspace and outputs."""

    def __init__(self, query, key, value, block_sparse_mask, *, num_heads: int,
                 num_key_value_heads: int = 0, scale_value: float = 1.0,
                 block_shape=(128, 128), input_layout: str = "BNSD",
                 actual_seq_lengths=None, actual_seq_lengths_kv=None,
                 softmax_lse_flag: bool = False, dequant_scale_query=None,
                 dequant_scale_key=None, dequant_scale_value=None, out=None, lse=None):
        self.plan = None
        if out is None:
            # FP8 inputs give a bf16 output
            odt = torch.bfloat16 if query.dtype == torch.float8_e4m3fn else query.dtype
            out = torch.empty(query.shape, dtype=odt, device=query.device)
        if softmax_lse_flag and lse is None:
            if input_layout == "TND":
                lse = torch.empty(query.shape[0], num_heads, 1, dtype=torch.float32,
                                  device=query.device)
            else:
                S = query.shape[2] if input_layout == "BNSD" else query.shape[1]
                lse = torch.empty(query.shape[0], num_heads, S, 1, dtype=torch.float32,
                                  device=query.device)
        self.out, self.lse = out, (lse if softmax_lse_flag else None)
        scales = (dequant_scale_query, dequant_scale_key, dequant_scale_value)
        self._keep = (query, key, value, block_sparse_mask, out, lse) + scales
        p = bsa_params()
        bsa_params_init(p)
        self._sdesc = [describe(t) for t in scales]
        p.dequant_scale_query, p.dequant_scale_key, p.dequant_scale_value = [
            ctypes.pointer(d) if d is not None else None for d in self._sdesc]
        self._layout = input_layout.encode()
        p.q_input_layout = self._layout
        p.kv_input_layout = self._layout
        p.num_heads = num_heads
        p.num_key_value_heads = num_key_value_heads
        p.scale_value = scale_value
        p.block_shape[0], p.block_shape[1] = block_shape
        qp, qn, qa = _host_i64(actual_seq_lengths)
        kp, kn, ka = _host_i64(actual_seq_lengths_kv)
        p.actual_seq_lengths, p.n_actual_seq_lengths = qp, qn
        p.actual_seq_lengths_kv, p.n_actual_seq_lengths_kv = kp, kn
        p.softmax_lse_flag = 1 if softmax_lse_flag else 0
        args = (describe(query), describe(key), describe(value), describe(block_sparse_mask), None,
                None, p, describe(out), describe(lse) if softmax_lse_flag else None)
        t0 = time.perf_counter()
        st, ws, plan = bsa_get_workspace_size(*args)
        self.phase1_s = time.perf_counter() - t0     # the C call alone (validation, plan, upload)
        del qa, ka
        if st != FIA_OK:
            raise FiaError(st, "bsa_get_workspace_size")
        self.plan = plan
        self.workspace_size = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
        self.device = query.device

    def run(self):
        st = bsa_run(self.workspace.data_ptr(), self.workspace_size, self.plan,
                     _stream_handle(self.device))
        if st != FIA_OK:
            raise FiaError(st, "bsa_run")
        return self.out, self.lse

    def run_noalloc(self):
        """Phase 2 on the library's static device scratch (fia_run_noalloc)."""
        st = fia_run_noalloc(self.plan, _stream_handle(self.device))
        if st != FIA_OK:
            raise FiaError(st, "fia_run_noalloc")
        return self.out, self.lse

    def schedule(self):
        """(cnt, idx) int32 tensors of the compacted schedule of the last run."""
        st, co, io, nqb, nkb = bsa_schedule_layout(self.plan)
        if st != FIA_OK:
            raise FiaError(st, "bsa_schedule_layout")
        rows = self.workspace[co:co + 4 * (self._rows(nqb))].view(torch.int32)
        idx = self.workspace[io:io + 4 * self._rows(nqb) * nkb].view(torch.int32)
        return rows, idx.view(-1, nkb), nqb, nkb

    def _rows(self, nqb):
        B = self._keep[3].shape[0]
        N = self._keep[3].shape[1]
        return B * N * nqb

    def close(self):
        if self.plan:
            fia_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fused_infer_attention_score(query, key, value, **kw):
    """One call of the fused inference attention: returns (attention_out,
    softmax_lse); softmax_lse is a shape-[1] zero tensor when not requested
    (outputs description of the v2 page)."""
    plan = FiaPlan(query, key, value, **kw)
    try:
        out, lse = plan.run()
    finally:
        plan.close()
    if lse is None:
        lse = torch.zeros(1, dtype=torch.float32, device=query.device)
    return out, lse


def block_sparse_attention(query, key, value, block_sparse_mask, **kw):
    plan = BsaPlan(query, key, value, block_sparse_mask, **kw)
    try:
        out, lse = plan.run()
    finally:
        plan.close()
    if lse is None:
        lse = torch.zeros(1, dtype=torch.float32, device=query.device)
    return out, lse
