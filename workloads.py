"""Seeded synthetic inputs for the fused inference attention forward.

This module only draws random numbers and lays them out: lengths, query/key/
value tensors, paged block tables, block-sparse masks.  It computes nothing of
the attention method itself.  Both the fp64 oracle (tests) and the HIP path
read the tensors it returns, so both sides see the same rounded values.

Recipe (one numpy SeedSequence per workload, spawned into six streams in a
fixed order: lengths, Q, K, V, block table / pool permutation, block mask):

* values: float32 standard normal, rounded to fp16/bf16 (round to nearest
  even, by torch's dtype conversion).  Large value tensors are drawn with a
  torch generator seeded from the stream, on the device they are meant for.
* padded layouts (BNSD/BSND) fill the padding with the same N(0,1) draws, or
  with NaN when ``nan_padding`` is set (a padding row must never be read).
* decode block tables take a seeded permutation of the physical pool
  consecutively; unused entries are -1.
* block-sparse masks: iid Bernoulli(p) per (q-block, kv-block), then the
  diagonal block forced on.

The five named workloads follow the workload list of the fused inference
attention pages' use cases (dense causal prefill, GQA causal prefill, paged GQA
decode, varlen TND prefill, block-sparse prefill).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

INT_MAX = 2147483647

STREAM_LENGTHS, STREAM_Q, STREAM_K, STREAM_V, STREAM_TABLE, STREAM_MASK = range(6)


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(6)


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def normal_tensor(shape, dtype: torch.dtype, ss: np.random.SeedSequence,
                  device: str = "cpu") -> torch.Tensor:
    """iid N(0,1) float32 draws rounded to ``dtype`` on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def int8_tensor(shape, ss: np.random.SeedSequence, device: str = "cpu") -> torch.Tensor:
    """iid integers uniform in [-127, 127] as int8 on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    return torch.randint(-127, 128, tuple(shape), generator=g, device=device, dtype=torch.int8)


@dataclass
class FiaCase:
    """One fused-infer-attention invocation with its inputs."""
    name: str
    layout: str                 # "BNSD" | "BSND" | "BSH" | "TND"
    dtype: torch.dtype
    B: int
    QN: int
    KVN: int
    Sq: int                     # padded query S (TND: total query rows T)
    Skv: int                    # padded kv S (TND: T_kv; paged: unused)
    Dqk: int
    Dv: int
    scale: float
    sparse_mode: int = 0
    pre_tokens: int = INT_MAX
    next_tokens: int = INT_MAX
    lq: Optional[np.ndarray] = None       # per-batch valid query lengths
    lkv: Optional[np.ndarray] = None      # per-batch valid kv lengths
    q: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    atten_mask: Optional[torch.Tensor] = None   # uint8/bool, nonzero = masked
    block_table: Optional[torch.Tensor] = None  # int32 [B, max_blocks]
    block_size: int = 0
    pool_layout: int = 0        # 0: (NB, KVN, bs, D)   1: (NB, bs, KVN*D)
    return_lse: bool = True
    meta: dict = field(default_factory=dict)
    # int8 key/value: {"dequant_scale_key": t, "dequant_scale_value": t,
    # "dequant_offset_key": t|None, "dequant_offset_value": t|None,
    # "key_quant_mode": 0|1, "value_quant_mode": 0|1}
    quant: Optional[dict] = None
    # MLA: {"query_rope": t, "key_rope": t}, laid out like query / key with D = 64
    rope: Optional[dict] = None

    @property
    def decode(self) -> bool:
        return self.layout != "TND" and self.Sq == 1

    def seq_qlen_arg(self):
        """actual_seq_qlen as the API takes it (cumulative for TND)."""
        if self.lq is None:
            return None
        if self.layout == "TND":
            return np.cumsum(self.lq).astype(np.int64)
        return self.lq.astype(np.int64)

    def seq_kvlen_arg(self):
        if self.lkv is None:
            return None
        if self.layout == "TND" and (self.block_table is None or self.rope is None):
            return np.cumsum(self.lkv).astype(np.int64)
        # (TND with page attention and a query D of 512, the MLA case: each
        # batch's own length)
        return self.lkv.astype(np.int64)


@dataclass
class BsaCase:
    """One block-sparse attention invocation with its inputs."""
    name: str
    layout: str                 # "BNSD" | "BSND" | "TND"
    dtype: torch.dtype
    B: int
    QN: int
    KVN: int
    Sq: int
    Skv: int
    D: int
    X: int
    Y: int
    scale: float
    lq: Optional[np.ndarray] = None
    lkv: Optional[np.ndarray] = None
    q: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    block_mask: Optional[torch.Tensor] = None   # uint8 [B, QN, nqb, nkb], nonzero = selected
    return_lse: bool = True
    meta: dict = field(default_factory=dict)
    # FP8 (E4M3FN) q/k/v: {"dequant_scale_query": [B, QN, nqb, 1],
    # "dequant_scale_key": [B, KVN, nkb, 1], "dequant_scale_value": ...} fp32
    fp8: Optional[dict] = None

    def seq_qlen_arg(self):
        if self.lq is None:
            return None
        if self.layout == "TND":
            return np.cumsum(self.lq).astype(np.int64)
        return self.lq.astype(np.int64)

    def seq_kvlen_arg(self):
        if self.lkv is None:
            return None
        if self.layout == "TND":
            return np.cumsum(self.lkv).astype(np.int64)
        return self.lkv.astype(np.int64)


def _shape(layout, B, N, S, D):
    if layout == "BNSD":
        return (B, N, S, D)
    if layout in ("BSND",):
        return (B, S, N, D)
    if layout == "BSH":
        return (B, S, N * D)
    if layout == "TND":
        return (S, N, D)
    raise ValueError(layout)


def _fill_padding_nan(t: torch.Tensor, layout: str, lens: np.ndarray, N: int, D: int):
    """Overwrite every row past a batch's valid length with NaN."""
    if layout == "TND":
        return t
    for b, L in enumerate(lens):
        L = int(L)
        if layout == "BNSD":
            t[b, :, L:, :] = float("nan")
        elif layout == "BSND":
            t[b, L:, :, :] = float("nan")
        elif layout == "BSH":
            t[b, L:, :] = float("nan")
    return t


def make_fia(name="custom", *, layout="BNSD", dtype=torch.bfloat16, B=1, QN=2, KVN=None,
             Sq=64, Skv=None, Dqk=64, Dv=None, scale=None, sparse_mode=0,
             pre_tokens=INT_MAX, next_tokens=INT_MAX, lq=None, lkv=None,
             mask_kind=None, seed=0, device="cpu", nan_padding=False,
             return_lse=True) -> FiaCase:
    """General contiguous-KV case.  ``lq``/``lkv`` are per-batch valid lengths
    (None = full).  For TND ``Sq``/``Skv`` are recomputed as the totals.
    ``mask_kind``: None, "template" (2048x2048 lower-triangular template for
    modes 2/3/4), "random" (iid 0/1 full mask), "zeros", or a callable
    (b, i, j) -> bool giving "masked"."""
    KVN = QN if KVN is None else KVN
    Skv = Sq if Skv is None else Skv
    Dv = Dqk if Dv is None else Dv
    scale = 1.0 / math.sqrt(Dqk) if scale is None else scale
    ss = _streams(seed)
    if lq is not None:
        lq = np.asarray(lq, dtype=np.int64)
    if lkv is not None:
        lkv = np.asarray(lkv, dtype=np.int64)
    if layout == "TND":
        assert lq is not None and lkv is not None
        Sq, Skv = int(lq.sum()), int(lkv.sum())
    q = normal_tensor(_shape(layout, B, QN, Sq, Dqk), dtype, ss[STREAM_Q], device)
    k = normal_tensor(_shape(layout, B, KVN, Skv, Dqk), dtype, ss[STREAM_K], device)
    v = normal_tensor(_shape(layout, B, KVN, Skv, Dv), dtype, ss[STREAM_V], device)
    if nan_padding and layout != "TND":
        if lq is not None:
            _fill_padding_nan(q, layout, lq, QN, Dqk)
        if lkv is not None:
            _fill_padding_nan(k, layout, lkv, KVN, Dqk)
            _fill_padding_nan(v, layout, lkv, KVN, Dv)
    mask = None
    if mask_kind == "template":
        mask = torch.triu(torch.ones(2048, 2048, dtype=torch.uint8), diagonal=1).to(device)
    elif mask_kind == "random":
        rng = np.random.default_rng(ss[STREAM_MASK])
        mask = torch.from_numpy(rng.integers(0, 2, size=(B, 1, Sq, Skv), dtype=np.uint8)).to(device)
    elif mask_kind == "zeros":
        mask = torch.zeros(B, 1, Sq, Skv, dtype=torch.uint8, device=device)
    elif callable(mask_kind):
        m = np.zeros((B, 1, Sq, Skv), dtype=np.uint8)
        for b in range(B):
            for i in range(Sq):
                for j in range(Skv):
                    m[b, 0, i, j] = 1 if mask_kind(b, i, j) else 0
        mask = torch.from_numpy(m).to(device)
    return FiaCase(name=name, layout=layout, dtype=dtype, B=B, QN=QN, KVN=KVN, Sq=Sq, Skv=Skv,
                   Dqk=Dqk, Dv=Dv, scale=scale, sparse_mode=sparse_mode,
                   pre_tokens=pre_tokens, next_tokens=next_tokens, lq=lq, lkv=lkv,
                   q=q, k=k, v=v, atten_mask=mask, return_lse=return_lse)


def make_paged_decode(name="custom", *, dtype=torch.bfloat16, B=2, QN=4, KVN=2, D=64,
                      lkv=(100, 37), block_size=16, pool_layout=0, scale=None, seed=0,
                      device="cpu", q_layout="BNSD", extra_blocks=0, table_cols=None,
                      return_lse=True, mask_p=None, mask_shape="B1S") -> FiaCase:
    """Paged decode: Q_S = 1, K/V in a shared physical pool addressed through a
    block table holding a seeded permutation of the pool's block ids.
    ``mask_p``: an atten_mask with iid Bernoulli(mask_p) masked kv tokens, of
    shape (B, KV_S) ("BS") or (B, 1, 1, KV_S) ("B1S"), KV_S = cols * block_size."""
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ss = _streams(seed)
    lkv = np.asarray(lkv, dtype=np.int64)
    nblk = [(int(L) + block_size - 1) // block_size for L in lkv]
    NB = sum(nblk) + extra_blocks
    cols = max(max(nblk), 1) if table_cols is None else table_cols
    rng = np.random.default_rng(ss[STREAM_TABLE])
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((B, cols), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    qshape = (B, QN, 1, D) if q_layout == "BNSD" else ((B, 1, QN, D) if q_layout == "BSND" else (B, 1, QN * D))
    q = normal_tensor(qshape, dtype, ss[STREAM_Q], device)
    pshape = (NB, KVN, block_size, D) if pool_layout == 0 else (NB, block_size, KVN * D)
    k = normal_tensor(pshape, dtype, ss[STREAM_K], device)
    v = normal_tensor(pshape, dtype, ss[STREAM_V], device)
    mask = None
    if mask_p is not None:
        mrng = np.random.default_rng(ss[STREAM_MASK])
        m = (mrng.random((B, cols * block_size)) < mask_p).astype(np.uint8)
        if mask_shape == "B1S":
            m = m.reshape(B, 1, 1, -1)
        mask = torch.from_numpy(np.ascontiguousarray(m)).to(device)
    return FiaCase(name=name, layout=q_layout, dtype=dtype, B=B, QN=QN, KVN=KVN, Sq=1,
                   Skv=cols * block_size, Dqk=D, Dv=D, scale=scale, lq=None, lkv=lkv,
                   q=q, k=k, v=v, atten_mask=mask, block_table=torch.from_numpy(table).to(device),
                   block_size=block_size, pool_layout=pool_layout, return_lse=return_lse,
                   meta={"NB": NB})


def make_paged_prefill(name="custom", *, layout="BNSD", dtype=torch.bfloat16, B=2, QN=4,
                       KVN=2, D=64, Sq=64, lq=None, lkv=(300, 170), block_size=128,
                       pool_layout=0, sparse_mode=3, pre_tokens=INT_MAX, next_tokens=INT_MAX,
                       mask_kind=None, scale=None, seed=0, device="cpu", extra_blocks=0,
                       table_cols=None, nan_pool=False, return_lse=True) -> FiaCase:
    """Prefill (query S > 1) against a paged KV cache: the query in ``layout``
    (BNSD/BSND/BSH, or TND with the batches' ``lq`` rows back to back) with
    per-batch lengths ``lq`` (None = Sq), K/V in a shared
    physical pool addressed through a block table holding a seeded
    permutation of the pool's block ids (unused entries -1).  ``nan_pool``
    fills the pool's unreferenced blocks and the tail rows of each batch's
    last block with NaN (they must never be read).  ``mask_kind`` as in
    :func:`make_fia` ("random"/"zeros" masks are [B, 1, Sq, cols * block_size])."""
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ss = _streams(seed)
    lkv = np.asarray(lkv, dtype=np.int64)
    if lq is not None:
        lq = np.asarray(lq, dtype=np.int64)
    nblk = [(int(L) + block_size - 1) // block_size for L in lkv]
    NB = sum(nblk) + extra_blocks
    cols = max(max(nblk), 1) if table_cols is None else table_cols
    rng = np.random.default_rng(ss[STREAM_TABLE])
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((B, cols), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    if layout == "TND":
        Sq = int(lq.sum())
    q = normal_tensor(_shape(layout, B, QN, Sq, D), dtype, ss[STREAM_Q], device)
    pshape = (NB, KVN, block_size, D) if pool_layout == 0 else (NB, block_size, KVN * D)
    k = normal_tensor(pshape, dtype, ss[STREAM_K], device)
    v = normal_tensor(pshape, dtype, ss[STREAM_V], device)
    if nan_pool:
        used = set(int(x) for x in table.reshape(-1) if x >= 0)
        for blk in range(NB):
            if blk not in used:
                k[blk] = float("nan")
                v[blk] = float("nan")
        for b in range(B):
            if nblk[b] == 0:
                continue
            last, tail = int(table[b, nblk[b] - 1]), int(lkv[b]) - (nblk[b] - 1) * block_size
            if pool_layout == 0:
                k[last, :, tail:] = float("nan")
                v[last, :, tail:] = float("nan")
            else:
                k[last, tail:] = float("nan")
                v[last, tail:] = float("nan")
    Skv = cols * block_size
    mask = None
    if mask_kind == "template":
        mask = torch.triu(torch.ones(2048, 2048, dtype=torch.uint8), diagonal=1).to(device)
    elif mask_kind == "random":
        mrng = np.random.default_rng(ss[STREAM_MASK])
        mask = torch.from_numpy(mrng.integers(0, 2, size=(B, 1, Sq, Skv), dtype=np.uint8)).to(device)
    elif mask_kind == "zeros":
        mask = torch.zeros(B, 1, Sq, Skv, dtype=torch.uint8, device=device)
    return FiaCase(name=name, layout=layout, dtype=dtype, B=B, QN=QN, KVN=KVN, Sq=Sq, Skv=Skv,
                   Dqk=D, Dv=D, scale=scale, sparse_mode=sparse_mode, pre_tokens=pre_tokens,
                   next_tokens=next_tokens, lq=lq, lkv=lkv, q=q, k=k, v=v, atten_mask=mask,
                   block_table=torch.from_numpy(table).to(device), block_size=block_size,
                   pool_layout=pool_layout, return_lse=return_lse, meta={"NB": NB})


def make_mla_decode(name="custom", *, layout="BSND", dtype=torch.bfloat16, B=2, QN=16, Sq=1,
                    lq=None, lkv=(100, 37), block_size=16, D=512, Dr=64, pool_layout=1,
                    scale=None, seed=0, device="cpu", extra_blocks=0, nan_pool=False,
                    return_lse=True, band=None) -> FiaCase:
    """MLA decode: query (``layout``, Q_N = QN, S = Sq <= 16, D = 512; TND: the
    batches' ``lq`` tokens back to back) with its 64-wide rope part, one kv head; key and value (D = 512) and key_rope
    (D = 64) in a shared paged pool, (NB, bs, D) (``pool_layout`` 1) or
    (NB, 1, bs, D) (0), addressed through a block table holding a seeded
    permutation of the pool's block ids.  Query S > 1 uses bottom-right causal
    masking (sparse_mode 3 with the 2048 template).  iid N(0,1) inputs; scale
    1/sqrt(D + Dr) unless given.  ``nan_pool`` fills the unreferenced blocks
    and the tail rows of each batch's last block with NaN.  ``band`` =
    (pre_tokens, next_tokens) selects sparse_mode 4 (bottom-right band, the
    2048 template as mask)."""
    scale = 1.0 / math.sqrt(D + Dr) if scale is None else scale
    ss = _streams(seed)
    lkv = np.asarray(lkv, dtype=np.int64)
    if lq is not None:
        lq = np.asarray(lq, dtype=np.int64)
    nblk = [(int(L) + block_size - 1) // block_size for L in lkv]
    NB = sum(nblk) + extra_blocks
    cols = max(max(nblk), 1)
    rng = np.random.default_rng(ss[STREAM_TABLE])
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((B, cols), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    sq, sqr = ss[STREAM_Q].spawn(2)
    sk, skr = ss[STREAM_K].spawn(2)
    if layout == "TND":
        # TND: the batches' query tokens (lq, each 1..16) back to back
        Sq = int(lq.sum())
    q = normal_tensor(_shape(layout, B, QN, Sq, D), dtype, sq, device)
    qr = normal_tensor(_shape(layout, B, QN, Sq, Dr), dtype, sqr, device)
    def pool(d):
        return (NB, 1, block_size, d) if pool_layout == 0 else (NB, block_size, d)
    k = normal_tensor(pool(D), dtype, sk, device)
    kr = normal_tensor(pool(Dr), dtype, skr, device)
    v = normal_tensor(pool(D), dtype, ss[STREAM_V], device)
    if nan_pool:
        used = set(int(x) for x in table.reshape(-1) if x >= 0)
        for t in (k, kr, v):
            for blk in range(NB):
                if blk not in used:
                    t[blk] = float("nan")
            for b in range(B):
                if nblk[b] == 0:
                    continue
                last, tail = int(table[b, nblk[b] - 1]), int(lkv[b]) - (nblk[b] - 1) * block_size
                if pool_layout == 0:
                    t[last, :, tail:] = float("nan")
                else:
                    t[last, tail:] = float("nan")
    mask = None
    causal = (lq.max() > 1) if layout == "TND" else Sq > 1
    if causal or band is not None:
        mask = torch.triu(torch.ones(2048, 2048, dtype=torch.uint8), diagonal=1).to(device)
    mode = 4 if band is not None else (3 if causal else 0)
    pre, nxt = band if band is not None else (INT_MAX, INT_MAX)
    return FiaCase(name=name, layout=layout, dtype=dtype, B=B, QN=QN, KVN=1, Sq=Sq,
                   Skv=cols * block_size, Dqk=D, Dv=D, scale=scale, sparse_mode=mode,
                   pre_tokens=pre, next_tokens=nxt,
                   lq=lq, lkv=lkv, q=q, k=k, v=v, atten_mask=mask,
                   block_table=torch.from_numpy(table).to(device), block_size=block_size,
                   pool_layout=pool_layout, return_lse=return_lse, meta={"NB": NB},
                   rope={"query_rope": qr, "key_rope": kr})


def make_quant_decode(name="custom", *, layout="BNSD", B=2, QN=4, KVN=2, D=64, Sq=1, Skv=None,
                      lkv=(100, 37), kmode=0, vmode=0, offsets=True, sparse_mode=0, scale=None,
                      seed=0, device="cpu", pow2=False, unit=False, return_lse=True,
                      block_size=0, pool_layout=0, extra_blocks=0) -> FiaCase:
    """Decode (query S <= 16) against an int8 KV cache (kv pseudo-quantization):
    bf16 query, int8 key/value uniform in [-127, 127], each value standing for
    scale * (x + offset).  Mode 0 (per channel): bf16 scale ~ U[0.004, 0.02],
    offset ~ U[-8, 8], shape [KV_N, D]; mode 1 (per token): fp32, shape
    [B, KV_S].  ``pow2``: scales 2^-k (k in 5..7) and integer offsets (the
    dequantized cache is then exact in bf16); ``unit``: scale 1, offset 0.
    ``block_size`` > 0: K/V are int8 pools (NB, KV_N, bs, D) (``pool_layout``
    0) or (NB, bs, KV_N * D) (1) addressed through a block table holding a
    seeded permutation of the pool's block ids (unused entries -1); KV_S of
    the per-token scales is then cols * bs."""
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ss = _streams(seed)
    lkv = np.asarray(lkv, dtype=np.int64)
    q = normal_tensor(_shape(layout, B, QN, Sq, D), torch.bfloat16, ss[STREAM_Q], device)
    table = None
    if block_size:
        nblk = [(int(L) + block_size - 1) // block_size for L in lkv]
        NB = sum(nblk) + extra_blocks
        cols = max(max(nblk), 1)
        rng = np.random.default_rng(ss[STREAM_TABLE])
        perm = rng.permutation(NB).astype(np.int32)
        table = np.full((B, cols), -1, dtype=np.int32)
        pos = 0
        for b in range(B):
            table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
            pos += nblk[b]
        Skv = cols * block_size
        kshape = (NB, KVN, block_size, D) if pool_layout == 0 else (NB, block_size, KVN * D)
    else:
        Skv = int(lkv.max()) if Skv is None else Skv
        kshape = _shape(layout, B, KVN, Skv, D)
    k = int8_tensor(kshape, ss[STREAM_K], device)
    v = int8_tensor(kshape, ss[STREAM_V], device)
    prng = np.random.default_rng(ss[STREAM_MASK])

    def params(mode):
        shp = (KVN, D) if mode == 0 else (B, Skv)
        dt = torch.bfloat16 if mode == 0 else torch.float32
        if unit:
            sc, of = np.ones(shp), np.zeros(shp)
        elif pow2:
            sc = 2.0 ** -prng.integers(5, 8, size=shp)
            of = prng.integers(-8, 9, size=shp).astype(np.float64)
        else:
            sc = prng.uniform(0.004, 0.02, size=shp)
            of = prng.uniform(-8.0, 8.0, size=shp)
        st = torch.from_numpy(sc).to(dt).to(device)
        ot = torch.from_numpy(of).to(dt).to(device) if offsets else None
        return st, ot

    ks, ko = params(kmode)
    vs, vo = params(vmode)
    quant = {"dequant_scale_key": ks, "dequant_scale_value": vs, "dequant_offset_key": ko,
             "dequant_offset_value": vo, "key_quant_mode": kmode, "value_quant_mode": vmode}
    mask = None
    if sparse_mode == 3 and Sq > 1:
        mask = torch.triu(torch.ones(2048, 2048, dtype=torch.uint8), diagonal=1).to(device)
    return FiaCase(name=name, layout=layout, dtype=torch.bfloat16, B=B, QN=QN, KVN=KVN, Sq=Sq,
                   Skv=Skv, Dqk=D, Dv=D, scale=scale, sparse_mode=sparse_mode, lq=None, lkv=lkv,
                   q=q, k=k, v=v, atten_mask=mask, return_lse=return_lse, quant=quant,
                   block_table=None if table is None else torch.from_numpy(table).to(device),
                   block_size=block_size, pool_layout=pool_layout)


def make_bsa(name="custom", *, layout="BNSD", dtype=torch.bfloat16, B=1, QN=2, KVN=1,
             Sq=256, Skv=None, D=64, X=128, Y=128, p=0.25, lq=None, lkv=None, scale=None,
             seed=0, device="cpu", mask_kind="bernoulli", return_lse=True) -> BsaCase:
    """Block-sparse case; ``mask_kind``: "bernoulli" (iid p, diagonal forced),
    "ones", "diag", "lower" (block lower-triangular), or an explicit array."""
    Skv = Sq if Skv is None else Skv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ss = _streams(seed)
    if lq is not None:
        lq = np.asarray(lq, dtype=np.int64)
    if lkv is not None:
        lkv = np.asarray(lkv, dtype=np.int64)
    if layout == "TND":
        Sq, Skv = int(lq.sum()), int(lkv.sum())
        maxq, maxkv = int(lq.max()), int(lkv.max())
    else:
        maxq, maxkv = Sq, Skv
    nqb, nkb = -(-maxq // X), -(-maxkv // Y)
    q = normal_tensor(_shape(layout, B, QN, Sq, D), dtype, ss[STREAM_Q], device)
    k = normal_tensor(_shape(layout, B, KVN, Skv, D), dtype, ss[STREAM_K], device)
    v = normal_tensor(_shape(layout, B, KVN, Skv, D), dtype, ss[STREAM_V], device)
    if isinstance(mask_kind, np.ndarray):
        m = mask_kind.astype(np.uint8)
    elif mask_kind == "bernoulli":
        rng = np.random.default_rng(ss[STREAM_MASK])
        m = (rng.random((B, QN, nqb, nkb)) < p).astype(np.uint8)
        for i in range(min(nqb, nkb)):
            m[:, :, i, i] = 1
    elif mask_kind == "ones":
        m = np.ones((B, QN, nqb, nkb), dtype=np.uint8)
    elif mask_kind == "diag":
        m = np.zeros((B, QN, nqb, nkb), dtype=np.uint8)
        for i in range(min(nqb, nkb)):
            m[:, :, i, i] = 1
    elif mask_kind == "lower":
        m = np.tril(np.ones((nqb, nkb), dtype=np.uint8))[None, None].repeat(B, 0).repeat(QN, 1)
    else:
        raise ValueError(mask_kind)
    return BsaCase(name=name, layout=layout, dtype=dtype, B=B, QN=QN, KVN=KVN, Sq=Sq, Skv=Skv,
                   D=D, X=X, Y=Y, scale=scale, lq=lq, lkv=lkv, q=q, k=k, v=v,
                   block_mask=torch.from_numpy(np.ascontiguousarray(m)).to(device),
                   return_lse=return_lse)


def _quantize_blocks(x: torch.Tensor, layout: str, blk: int, pow2: bool):
    """Per-(batch, head, row block) E4M3FN quantization of a BNSD/BSND tensor:
    scale = amax / 448 of the block (a power of two at or above it with
    ``pow2``), values x / scale rounded to E4M3FN.  Returns (fp8 tensor,
    fp32 scales [B, N, nblk, 1])."""
    xb = x if layout == "BNSD" else x.permute(0, 2, 1, 3)
    B, N, S, D = xb.shape
    nb = -(-S // blk)
    pad = torch.zeros(B, N, nb * blk, D, dtype=torch.float32, device=x.device)
    pad[:, :, :S] = xb
    amax = pad.reshape(B, N, nb, blk * D).abs().amax(dim=-1).clamp(min=1e-6)
    sc = amax / 448.0
    if pow2:
        sc = torch.exp2(torch.ceil(torch.log2(sc)))
    q = (pad.reshape(B, N, nb, blk, D) / sc[..., None, None]).reshape(B, N, nb * blk, D)[:, :, :S]
    q = q.to(torch.float8_e4m3fn)
    if layout != "BNSD":
        q = q.permute(0, 2, 1, 3)
    return q.contiguous(), sc[..., None].contiguous()


def make_bsa_fp8(name="custom", *, layout="BNSD", B=1, QN=2, KVN=1, Sq=256, Skv=None, D=128,
                 Y=256, p=0.25, lq=None, lkv=None, scale=None, seed=0, device="cpu",
                 mask_kind="bernoulli", pow2=False, return_lse=True) -> BsaCase:
    """Block-sparse case with FP8 (E4M3FN) query / key / value: fp32 N(0,1)
    draws quantized per block (query 128-row blocks, key / value Y-token
    blocks, Y = 256 or 512) with scale = block amax / 448.  Mask iid
    Bernoulli(p) per (q block, kv block) with the kv block holding the q
    block's diagonal forced on ("ones": all selected)."""
    X = 128
    Skv = Sq if Skv is None else Skv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    ss = _streams(seed)
    if lq is not None:
        lq = np.asarray(lq, dtype=np.int64)
    if lkv is not None:
        lkv = np.asarray(lkv, dtype=np.int64)
    nqb, nkb = -(-Sq // X), -(-Skv // Y)
    qf = normal_tensor(_shape(layout, B, QN, Sq, D), torch.float32, ss[STREAM_Q], device)
    kf = normal_tensor(_shape(layout, B, KVN, Skv, D), torch.float32, ss[STREAM_K], device)
    vf = normal_tensor(_shape(layout, B, KVN, Skv, D), torch.float32, ss[STREAM_V], device)
    q, qs = _quantize_blocks(qf, layout, X, pow2)
    k, ks = _quantize_blocks(kf, layout, Y, pow2)
    v, vs = _quantize_blocks(vf, layout, Y, pow2)
    del qf, kf, vf
    if mask_kind == "ones":
        m = np.ones((B, QN, nqb, nkb), dtype=np.uint8)
    else:
        rng = np.random.default_rng(ss[STREAM_MASK])
        m = (rng.random((B, QN, nqb, nkb)) < p).astype(np.uint8)
        for i in range(nqb):
            if (i * X) // Y < nkb:
                m[:, :, i, (i * X) // Y] = 1
    return BsaCase(name=name, layout=layout, dtype=torch.float8_e4m3fn, B=B, QN=QN, KVN=KVN,
                   Sq=Sq, Skv=Skv, D=D, X=X, Y=Y, scale=scale, lq=lq, lkv=lkv, q=q, k=k, v=v,
                   block_mask=torch.from_numpy(np.ascontiguousarray(m)).to(device),
                   return_lse=return_lse,
                   fp8={"dequant_scale_query": qs, "dequant_scale_key": ks,
                        "dequant_scale_value": vs})


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

def c1_dense_causal_fp16(device="cpu") -> FiaCase:
    """B=1, Q_N=KV_N=2, S=128, D=64, fp16, BNSD, causal (sparse_mode 3 with the
    2048x2048 lower-triangular template), scale 1/8, LSE on."""
    return make_fia("dense_causal_prefill_fp16_b1_n2_s128_d64", layout="BNSD",
                    dtype=torch.float16, B=1, QN=2, KVN=2, Sq=128, Dqk=64,
                    scale=1.0 / 8.0, sparse_mode=3, mask_kind="template", seed=1001,
                    device=device)


def c2_lengths():
    rng = np.random.default_rng(_streams(1002)[STREAM_LENGTHS])
    return rng.integers(1024, 4096, size=4, endpoint=True).astype(np.int64)


def c2_gqa_causal_bf16(device="cpu", nan_padding=False) -> FiaCase:
    """B=4, Q_N=32, KV_N=8, max S=4096, D=128, bf16, BSND, per-batch
    actual_seq_qlen = actual_seq_kvlen ~ U{1024..4096}, causal (mode 3)."""
    L = c2_lengths()
    return make_fia("gqa_causal_prefill_bf16_b4_n32_kv8_s4096_d128", layout="BSND",
                    dtype=torch.bfloat16, B=4, QN=32, KVN=8, Sq=4096, Dqk=128,
                    scale=1.0 / math.sqrt(128), sparse_mode=3, mask_kind="template",
                    lq=L, lkv=L, seed=1002, device=device, nan_padding=nan_padding)


def c3_lengths():
    rng = np.random.default_rng(_streams(1003)[STREAM_LENGTHS])
    return rng.integers(512, 32768, size=64, endpoint=True).astype(np.int64)


def c3_paged_decode_bf16(device="cpu") -> FiaCase:
    """B=64, Q_S=1, Q_N=32, KV_N=8, D=128, bf16, KV lengths ~ U{512..32768},
    page 128 tokens, pool layout (NB, KV_N, 128, 128), LSE on."""
    L = c3_lengths()
    return make_paged_decode("paged_gqa_decode_bf16_b64_n32_kv8_d128_bs128", dtype=torch.bfloat16,
                             B=64, QN=32, KVN=8, D=128, lkv=L, block_size=128, pool_layout=0,
                             seed=1003, device=device)


def c4_lengths():
    rng = np.random.default_rng(_streams(1004)[STREAM_LENGTHS])
    x = np.exp(rng.normal(math.log(1024.0), 1.0, size=16))
    return np.clip(np.rint(x), 64, 8192).astype(np.int64)


def c4_varlen_tnd_bf16(device="cpu") -> FiaCase:
    """16 sequences, lengths lognormal(median 1024, sigma 1) clipped to
    [64, 8192], TND, Q_N=KV_N=16, D_qk=192, D_v=128, causal, bf16."""
    L = c4_lengths()
    return make_fia("varlen_tnd_prefill_bf16_16seq_n16_d192_dv128", layout="TND",
                    dtype=torch.bfloat16, B=16, QN=16, KVN=16, Dqk=192, Dv=128,
                    scale=1.0 / math.sqrt(192), sparse_mode=3, mask_kind="template",
                    lq=L, lkv=L, seed=1004, device=device)


def c5_block_sparse_bf16(device="cpu") -> BsaCase:
    """B=1, Q_N=32, KV_N=8, S=32768, D=128, BNSD, block [128,128], mask
    Bernoulli(0.25) with the diagonal forced on, bf16, LSE on."""
    return make_bsa("block_sparse_prefill_bf16_b1_n32_kv8_s32768_d128", layout="BNSD",
                    dtype=torch.bfloat16, B=1, QN=32, KVN=8, Sq=32768, D=128, X=128, Y=128,
                    p=0.25, seed=1005, device=device)


def paged_prefill_lengths():
    rng = np.random.default_rng(_streams(1006)[STREAM_LENGTHS])
    lq = rng.integers(512, 2048, size=8, endpoint=True).astype(np.int64)
    hist = rng.integers(0, 14336, size=8, endpoint=True).astype(np.int64)
    return lq, lq + hist


def paged_chunked_prefill_bf16(device="cpu") -> FiaCase:
    """Chunked prefill against a paged cache: B=8, Q_N=32, KV_N=8, D=128,
    bf16, query BSND padded to 2048 rows with chunk lengths ~ U{512..2048},
    KV lengths = chunk + history ~ U{0..14336}, page 128 tokens, pool
    (NB, 128, KV_N * D), bottom-right causal (sparse_mode 3), LSE on."""
    lq, lkv = paged_prefill_lengths()
    return make_paged_prefill("paged_chunked_prefill_bf16_b8_n32_kv8_d128_bs128", layout="BSND",
                              dtype=torch.bfloat16, B=8, QN=32, KVN=8, D=128, Sq=2048, lq=lq,
                              lkv=lkv, block_size=128, pool_layout=1, sparse_mode=3,
                              mask_kind="template", seed=1006, device=device)


def paged_mtp_decode_bf16(device="cpu") -> FiaCase:
    """Multi-token decode (4 query tokens per sequence) against a paged cache:
    B=64, Q_S=4, Q_N=32, KV_N=8, D=128, bf16, BNSD, KV lengths ~ U{512..32768},
    page 128 tokens, pool (NB, KV_N, 128, 128), bottom-right causal, LSE on."""
    rng = np.random.default_rng(_streams(1007)[STREAM_LENGTHS])
    lkv = rng.integers(512, 32768, size=64, endpoint=True).astype(np.int64)
    return make_paged_prefill("paged_mtp4_decode_bf16_b64_n32_kv8_d128_bs128", layout="BNSD",
                              dtype=torch.bfloat16, B=64, QN=32, KVN=8, D=128, Sq=4, lq=None,
                              lkv=lkv, block_size=128, pool_layout=0, sparse_mode=3,
                              mask_kind="template", seed=1007, device=device)


def int8_kv_decode_bf16(device="cpu") -> FiaCase:
    """Decode against an int8 KV cache with per-channel scales and offsets:
    B=64, Q_S=1, Q_N=32, KV_N=8, D=128, bf16 query, BNSD, contiguous int8
    K/V [64, 8, 32768, 128], KV lengths ~ U{512..32768}, LSE on."""
    rng = np.random.default_rng(_streams(1008)[STREAM_LENGTHS])
    lkv = rng.integers(512, 32768, size=64, endpoint=True).astype(np.int64)
    return make_quant_decode("int8_kv_decode_perchannel_b64_n32_kv8_d128", layout="BNSD", B=64,
                             QN=32, KVN=8, D=128, Skv=32768, lkv=lkv, kmode=0, vmode=0,
                             seed=1008, device=device)


def int8_paged_decode_bf16(device="cpu") -> FiaCase:
    """Decode against a paged int8 KV cache with per-channel scales and
    offsets: the paged GQA decode shape (B=64, Q_S=1, Q_N=32, KV_N=8, D=128,
    its KV lengths ~ U{512..32768}), bf16 query, int8 pools
    (NB, KV_N, 128, 128) addressed through a seeded permutation, LSE on."""
    return make_quant_decode("int8_paged_decode_perchannel_b64_n32_kv8_d128_bs128", layout="BNSD",
                             B=64, QN=32, KVN=8, D=128, lkv=c3_lengths(), kmode=0, vmode=0,
                             block_size=128, pool_layout=0, seed=1011, device=device)


def fp8_block_sparse(device="cpu") -> BsaCase:
    """Block-sparse prefill with FP8 (E4M3FN) inputs: B=1, Q_N=32, KV_N=8,
    S=32768, D=128, BNSD, block [128, 256] (the quantization blocks), mask
    Bernoulli(0.25) with the diagonal's kv block forced on, per-block amax
    scales, bf16 output, LSE on."""
    return make_bsa_fp8("fp8_block_sparse_prefill_b1_n32_kv8_s32768_d128_y256", layout="BNSD",
                        B=1, QN=32, KVN=8, Sq=32768, D=128, Y=256, p=0.25, seed=1009,
                        device=device)


def mla_decode_bf16(device="cpu") -> FiaCase:
    """MLA decode: B=64, Q_S=1, Q_N=128, one kv head, D=512 + rope 64, bf16,
    BSND query, KV lengths ~ U{512..16384}, page 128 tokens, pools
    (NB, 128, 512) for key and value and (NB, 128, 64) for key_rope, LSE on."""
    rng = np.random.default_rng(_streams(1010)[STREAM_LENGTHS])
    lkv = rng.integers(512, 16384, size=64, endpoint=True).astype(np.int64)
    return make_mla_decode("mla_decode_bf16_b64_n128_d512_rope64_bs128", layout="BSND",
                           dtype=torch.bfloat16, B=64, QN=128, Sq=1, lkv=lkv, block_size=128,
                           pool_layout=1, seed=1010, device=device)


def mla_decode_shared_kv_bf16(device="cpu") -> FiaCase:
    """The MLA decode workload with value passed as the key tensor itself (the
    latent cache read as both key and value): key pool (NB, 128, 512) and
    key_rope pool (NB, 128, 64) only."""
    case = mla_decode_bf16(device)
    case.name = "mla_decode_shared_kv_bf16_b64_n128_d512_rope64_bs128"
    case.v = case.k
    case.meta["v_is_k"] = True
    return case


WORKLOADS = {
    "c1": c1_dense_causal_fp16,
    "c2": c2_gqa_causal_bf16,
    "c3": c3_paged_decode_bf16,
    "c4": c4_varlen_tnd_bf16,
    "c5": c5_block_sparse_bf16,
    "paged_prefill": paged_chunked_prefill_bf16,
    "mtp_decode": paged_mtp_decode_bf16,
    "int8_decode": int8_kv_decode_bf16,
    "int8_paged_decode": int8_paged_decode_bf16,
    "fp8_bsa": fp8_block_sparse,
    "mla_decode": mla_decode_bf16,
    "mla_shared_kv": mla_decode_shared_kv_bf16,
}
