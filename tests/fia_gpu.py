"""Helpers of the GPU tests: run a workload case through the C ABI on
cuda:0 and compare with the oracle at the tolerances of the workload
statement (max-abs 2e-2 bf16, 5e-3 fp16, 1e-3 for the fp32 LSE)."""
import sys

import numpy as np
import torch

import attention_fia_fwd_amd as fia

TOL_OUT = {torch.bfloat16: 2e-2, torch.float16: 5e-3}
TOL_LSE = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(case, device="cuda"):
    for name in ("q", "k", "v", "atten_mask", "block_table", "block_mask"):
        t = getattr(case, name, None)
        if t is not None and t.device.type != "cuda":
            setattr(case, name, t.to(device))
    for extra in ("quant", "fp8", "rope"):
        d = getattr(case, extra, None)
        if d:
            for key, t in d.items():
                if isinstance(t, torch.Tensor) and t.device.type != "cuda":
                    d[key] = t.to(device)
    return case


def fia_plan(case, **over):
    kw = dict(num_heads=case.QN, num_key_value_heads=case.KVN, softmax_scale=case.scale,
              input_layout=case.layout, sparse_mode=case.sparse_mode,
              pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
              return_softmax_lse=case.return_lse)
    if case.block_table is not None:
        kw.update(block_table=case.block_table, block_size=case.block_size)
    if case.atten_mask is not None:
        kw["atten_mask"] = case.atten_mask
    ql, kl = case.seq_qlen_arg(), case.seq_kvlen_arg()
    if ql is not None and not case.decode:
        kw["actual_seq_qlen"] = ql
    if kl is not None:
        kw["actual_seq_kvlen"] = kl
    if getattr(case, "quant", None):
        kw.update(case.quant)
    if getattr(case, "rope", None):
        kw.update(case.rope)
    kw.update(over)
    return fia.FiaPlan(case.q, case.k, case.v, **kw)


def bsa_plan(case, **over):
    kw = dict(num_heads=case.QN, num_key_value_heads=case.KVN, scale_value=case.scale,
              block_shape=(case.X, case.Y), input_layout=case.layout,
              softmax_lse_flag=case.return_lse)
    ql, kl = case.seq_qlen_arg(), case.seq_kvlen_arg()
    if ql is not None:
        kw["actual_seq_lengths"] = ql
        kw["actual_seq_lengths_kv"] = kl
    if getattr(case, "fp8", None):
        kw.update(case.fp8)
    kw.update(over)
    return fia.BsaPlan(case.q, case.k, case.v, case.block_mask, **kw)


def run(plan):
    out, lse = plan.run()
    torch.cuda.synchronize()
    return out, lse


def out_as_oracle_layout(case, out):
    """GPU output (query layout, BSH as [B,S,H]) as float64 numpy in the
    oracle's layout (BSH -> BSND)."""
    o = out.detach().float().cpu().to(torch.float64).numpy()
    if case.layout == "BSH":
        o = o.reshape(o.shape[0], o.shape[1], case.QN, -1)
    return o


def lse_as_oracle_layout(case, lse):
    l = lse.detach().cpu().to(torch.float64).numpy()
    return l[..., 0]


def compare(case, out, lse, ref_out, ref_lse, dtype=None):
    """Element-wise comparison; +inf LSE and exact-zero rows must match
    exactly.  Returns (max out err, max lse err)."""
    dtype = dtype or case.dtype
    if dtype == torch.float8_e4m3fn:
        dtype = torch.bfloat16               # FP8 inputs give a bf16 output
    o = out_as_oracle_layout(case, out)
    assert o.shape == ref_out.shape, (o.shape, ref_out.shape)
    assert np.all(np.isfinite(o)), "non-finite output"
    err = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    assert err <= TOL_OUT[dtype], f"{case.name}: max |out - oracle| = {err}"
    lerr = 0.0
    if lse is not None and ref_lse is not None:
        l = lse_as_oracle_layout(case, lse)
        assert l.shape == ref_lse.shape, (l.shape, ref_lse.shape)
        inf_ref = np.isinf(ref_lse)
        assert np.array_equal(np.isposinf(l), inf_ref), f"{case.name}: +inf rows differ"
        if (~inf_ref).any():
            lerr = float(np.max(np.abs(l[~inf_ref] - ref_lse[~inf_ref])))
        assert lerr <= TOL_LSE, f"{case.name}: max |lse - oracle| = {lerr}"
        zero_rows = inf_ref
        if zero_rows.any():
            # rows without any allowed key are exactly zero
            if case.layout == "TND":
                assert np.all(o[zero_rows] == 0)
            elif case.layout == "BNSD":
                assert np.all(o[zero_rows] == 0)
            else:
                assert np.all(o.transpose(0, 2, 1, 3)[zero_rows] == 0)
    return err, lerr


def sample_rows(case, n, seed=0, decode=False):
    """(b, h, i) triples spread over batches, heads and rows incl. the ends."""
    rng = np.random.default_rng(seed)
    B, QN = case.B, case.QN
    lq = np.ones(B, dtype=np.int64) if decode else (case.lq if case.lq is not None else np.full(B, case.Sq))
    rows = []
    for b in range(B):
        L = int(lq[b])
        if L == 0:
            continue
        for i in {0, L - 1, L // 2}:
            rows.append((b, int(rng.integers(QN)), i))
    while len(rows) < n:
        b = int(rng.integers(B))
        L = int(lq[b])
        if L:
            rows.append((b, int(rng.integers(QN)), int(rng.integers(L))))
    return rows[:max(n, len(rows))]


def gather_rows(case, out, lse, rows):
    o = out_as_oracle_layout(case, out)
    l = lse_as_oracle_layout(case, lse) if lse is not None else None
    go, gl = [], []
    starts = None
    if case.layout == "TND":
        starts = np.concatenate([[0], np.cumsum(case.lq)[:-1]])
    for b, h, i in rows:
        if case.layout == "TND":
            r = starts[b] + i
            go.append(o[r, h])
            gl.append(l[r, h] if l is not None else 0)
        elif case.layout == "BNSD":
            go.append(o[b, h, i])
            gl.append(l[b, h, i] if l is not None else 0)
        else:
            go.append(o[b, i, h])
            gl.append(l[b, h, i] if l is not None else 0)
    return np.array(go), np.array(gl)


def head_rows(case, heads, batches=None):
    """Every (b, h, i) of the given query heads (and batches, default all):
    whole heads of the output, each row below its batch's query length."""
    lq = np.ones(case.B, dtype=np.int64) if getattr(case, "decode", False) else (
        case.lq if case.lq is not None else np.full(case.B, case.Sq))
    bs = range(case.B) if batches is None else batches
    return [(b, h, i) for b in bs for h in heads for i in range(int(lq[b]))]


def seeded_subset(n, k, seed):
    """k distinct indices of range(n), sorted, from a seeded generator."""
    rng = np.random.default_rng(seed)
    return sorted(int(x) for x in rng.choice(n, size=min(k, n), replace=False))


def compare_rows(case, out, lse, rows, ref_o, ref_l, dtype=None):
    """Element-wise comparison of the listed rows (ref_o [n, Dv], ref_l [n])
    at the output / LSE tolerances; +inf rows must match exactly and hold
    out = 0.  Returns (max out err, max lse err)."""
    dtype = dtype or case.dtype
    if dtype == torch.float8_e4m3fn:
        dtype = torch.bfloat16
    go, gl = gather_rows(case, out, lse, rows)
    assert np.all(np.isfinite(go)), "non-finite output"
    err = float(np.max(np.abs(go - ref_o))) if go.size else 0.0
    assert err <= TOL_OUT[dtype], f"{case.name}: max |out - oracle| = {err}"
    lerr = 0.0
    if lse is not None:
        inf_ref = np.isinf(ref_l)
        assert np.array_equal(np.isposinf(gl), inf_ref), f"{case.name}: +inf rows differ"
        if (~inf_ref).any():
            lerr = float(np.max(np.abs(gl[~inf_ref] - ref_l[~inf_ref])))
        assert lerr <= TOL_LSE, f"{case.name}: max |lse - oracle| = {lerr}"
        assert np.all(go[inf_ref] == 0)
    return err, lerr
