"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant the pages
state, a textbook/library routine, or brute force on tiny inputs, so that a
plausible mistake in it (dropped term, wrong sign or index, transposed
operand, wrong mask alignment) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

INT_MAX = W.INT_MAX


# ---------------------------------------------------------------------------
# helpers: an independent dense reference built from library routines
# ---------------------------------------------------------------------------

def _to_bnsd64(t, layout, B, N, S, D, lens=None):
    """Per-batch float64 [N, L_b, D] views of a tensor in any layout."""
    t = t.detach().cpu().to(torch.float64)
    out = []
    if layout == "TND":
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        for b in range(B):
            out.append(t[starts[b]:starts[b] + lens[b]].permute(1, 0, 2))
        return out
    if layout == "BSH":
        t = t.reshape(B, S, N, D)
        layout = "BSND"
    if layout == "BSND":
        t = t.permute(0, 2, 1, 3)
    for b in range(B):
        L = S if lens is None else int(lens[b])
        out.append(t[b, :, :L])
    return out


def _keep_matrix(mode, Lq, Lkv, pre, nxt, mask_b=None):
    """Boolean keep-matrix via numpy tril/triu (library band routines)."""
    ones = np.ones((Lq, Lkv), dtype=bool)
    d = Lkv - Lq
    if mode == 0:
        if mask_b is None:
            return ones
        keep = (mask_b[:Lq, :Lkv] == 0)
        return keep & np.tril(ones, min(nxt, Lkv)) & np.triu(ones, -min(pre, Lq))
    if mode == 1:
        return mask_b[:Lq, :Lkv] == 0
    if mode == 2:
        return np.tril(ones, 0)
    if mode == 3:
        return np.tril(ones, d)
    if mode == 4:
        return np.tril(ones, min(nxt, Lkv) + d) & np.triu(ones, d - min(pre, Lq + Lkv))
    raise ValueError(mode)


def dense_reference(case):
    """softmax(scale*Q K^T + additive mask) V with torch float64 and
    logsumexp, per batch; GQA by repeat_interleave.  Returns lists per batch of
    [QN, Lq, Dv] outputs and [QN, Lq] lse (empty rows -> 0 / +inf)."""
    B, QN, KVN = case.B, case.QN, case.KVN
    lq = case.lq if case.lq is not None else np.full(B, case.Sq)
    lkv = case.lkv if case.lkv is not None else np.full(B, case.Skv)
    qs = _to_bnsd64(case.q, case.layout, B, QN, case.Sq, case.Dqk, lq if case.layout == "TND" or case.lq is not None else None)
    ks = _to_bnsd64(case.k, case.layout, B, KVN, case.Skv, case.Dqk, lkv if case.layout == "TND" or case.lkv is not None else None)
    vs = _to_bnsd64(case.v, case.layout, B, KVN, case.Skv, case.Dv, lkv if case.layout == "TND" or case.lkv is not None else None)
    mask = None
    if case.atten_mask is not None and case.sparse_mode in (0, 1):
        m = case.atten_mask.cpu().numpy()
        mask = m.reshape((-1,) + m.shape[-2:])
    outs, lses = [], []
    for b in range(B):
        Lq, Lkv = int(lq[b]), int(lkv[b])
        mb = None if mask is None else mask[b if mask.shape[0] > 1 else 0]
        keep = torch.from_numpy(_keep_matrix(case.sparse_mode, Lq, Lkv, case.pre_tokens,
                                             case.next_tokens, mb))
        k = ks[b].repeat_interleave(QN // KVN, dim=0)
        v = vs[b].repeat_interleave(QN // KVN, dim=0)
        s = case.scale * torch.matmul(qs[b][:, :Lq], k.transpose(1, 2))
        s = s.masked_fill(~keep, float("-inf"))
        lse = torch.logsumexp(s, dim=-1)
        p = torch.softmax(s, dim=-1)
        o = torch.matmul(torch.nan_to_num(p, nan=0.0), v)
        empty = ~keep.any(dim=-1)
        o[:, empty] = 0.0
        lse[:, empty] = float("inf")
        outs.append(o.numpy())
        lses.append(lse.numpy())
    return outs, lses


def oracle_per_batch(case, out, lse):
    """Split oracle outputs into per-batch [QN, Lq, Dv] / [QN, Lq]."""
    B = case.B
    lq = case.lq if case.lq is not None else np.full(B, case.Sq)
    res_o, res_l = [], []
    if case.layout == "TND":
        starts = np.concatenate([[0], np.cumsum(lq)[:-1]])
        for b in range(B):
            sl = slice(starts[b], starts[b] + lq[b])
            res_o.append(out[sl].transpose(1, 0, 2))
            res_l.append(lse[sl].T)
        return res_o, res_l
    for b in range(B):
        L = int(lq[b])
        o = out[b] if case.layout == "BNSD" else out[b].transpose(1, 0, 2)
        res_o.append(o[:, :L])
        res_l.append(lse[b][:, :L])
    return res_o, res_l


def assert_matches_reference(case, tol=1e-11):
    out, lse = oracle.attention(case)
    ro, rl = dense_reference(case)
    oo, ol = oracle_per_batch(case, out, lse)
    for b in range(case.B):
        np.testing.assert_allclose(oo[b], ro[b], atol=tol, rtol=0)
        both_inf = np.isinf(ol[b]) & np.isinf(rl[b])
        assert np.array_equal(np.isinf(ol[b]), np.isinf(rl[b]))
        np.testing.assert_allclose(ol[b][~both_inf], rl[b][~both_inf], atol=tol, rtol=0)
    return out, lse


# ---------------------------------------------------------------------------
# element reader
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_half_reader_is_exact_for_every_bit_pattern(dtype):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(dtype).to(torch.float64).numpy()
    got = np.array([oracle.read_half(int(b), dtype) for b in bits])
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(got[finite], ref[finite])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(np.isposinf(got), np.isposinf(ref))


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_zero_query_gives_mean_of_allowed_values_and_log_count():
    case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, KVN=1, Sq=9, Skv=13,
                      Dqk=16, Dv=8, sparse_mode=3, lq=[9, 5], lkv=[13, 11], seed=3)
    case.q.zero_()
    out, lse = oracle.attention(case)
    v = case.v.to(torch.float64).numpy()
    for b in range(2):
        Lq, Lkv = int(case.lq[b]), int(case.lkv[b])
        d = Lkv - Lq
        for h in range(2):
            for i in range(Lq):
                n = i + d + 1                      # keys j <= i + delta
                np.testing.assert_allclose(out[b, h, i], v[b, 0, :n].mean(0), atol=1e-12)
                assert lse[b, h, i] == pytest.approx(math.log(n), abs=1e-12)


def test_identical_keys_give_mean_of_values():
    case = W.make_fia(layout="BSND", dtype=torch.float16, B=1, QN=3, Sq=7, Dqk=32, seed=4)
    case.k[:] = case.k[:, :1]                      # every key equal to key 0
    out, _ = oracle.attention(case)
    v = case.v.to(torch.float64).numpy()
    for h in range(3):
        np.testing.assert_allclose(out[0, :, h], np.broadcast_to(v[0, :, h].mean(0), (7, 32)),
                                   atol=1e-12)


def test_single_key_returns_that_value_exactly():
    # causal row 0 sees only key 0; band pre=next=0 sees only key i + delta
    case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=1, QN=2, Sq=6, Skv=9, Dqk=16,
                      sparse_mode=4, pre_tokens=0, next_tokens=0, lq=[6], lkv=[9], seed=5)
    out, _ = oracle.attention(case)
    v = case.v.to(torch.float64).numpy()
    for h in range(2):
        for i in range(6):
            np.testing.assert_array_equal(out[0, h, i], v[0, h, i + 3])
    case3 = W.make_fia(layout="BNSD", dtype=torch.float16, B=1, QN=2, Sq=8, Dqk=16,
                       sparse_mode=3, seed=6)
    out3, _ = oracle.attention(case3)
    np.testing.assert_array_equal(out3[0, :, 0], case3.v.to(torch.float64).numpy()[0, :, 0])


def test_two_keys_follow_the_logistic_form():
    case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=1, QN=1, Sq=2, Dqk=8,
                      sparse_mode=2, scale=0.37, seed=7)
    out, lse = oracle.attention(case)
    q = case.q.to(torch.float64).numpy()[0, 0, 1]
    k = case.k.to(torch.float64).numpy()[0, 0]
    v = case.v.to(torch.float64).numpy()[0, 0]
    s0, s1 = 0.37 * float(q @ k[0]), 0.37 * float(q @ k[1])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    np.testing.assert_allclose(out[0, 0, 1], sig(s0 - s1) * v[0] + sig(s1 - s0) * v[1], atol=1e-12)
    assert lse[0, 0, 1] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), abs=1e-12)


def test_lse_equals_brute_force_log_of_sum():
    case = W.make_fia(layout="BNSD", dtype=torch.float16, B=1, QN=2, Sq=5, Skv=40, Dqk=16,
                      lq=[5], lkv=[40], sparse_mode=0, seed=8, scale=0.9)
    _, lse = oracle.attention(case)
    q = case.q.to(torch.float64).numpy()[0]
    k = case.k.to(torch.float64).numpy()[0]
    for h in range(2):
        for i in range(5):
            s = [0.9 * float(np.dot(q[h, i], k[h, j])) for j in range(40)]
            assert lse[0, h, i] == pytest.approx(math.log(math.fsum(math.exp(x) for x in s)), abs=1e-12)


# ---------------------------------------------------------------------------
# textbook cross-check for every mask mode, layout, dtype, GQA
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["BNSD", "BSND", "BSH"])
@pytest.mark.parametrize("mode", [0, 2, 3, 4])
def test_matches_torch_float64_softmax(layout, mode):
    case = W.make_fia(layout=layout, dtype=torch.bfloat16, B=2, QN=4, KVN=2, Sq=11, Skv=17,
                      Dqk=16, Dv=8 if layout != "BSH" else 16, sparse_mode=mode,
                      pre_tokens=3, next_tokens=2, lq=[11, 6], lkv=[17, 9], seed=10 + mode)
    assert_matches_reference(case)


@pytest.mark.parametrize("mode", [0, 1])
def test_explicit_mask_modes(mode):
    case = W.make_fia(layout="BNSD", dtype=torch.float16, B=2, QN=2, Sq=12, Skv=15, Dqk=8,
                      sparse_mode=mode, pre_tokens=4, next_tokens=1, lq=[12, 9], lkv=[15, 10],
                      mask_kind="random", seed=20 + mode)
    assert_matches_reference(case)


def test_tnd_matches_reference_and_per_sequence_runs():
    L = [5, 1, 12, 7]
    case = W.make_fia(layout="TND", dtype=torch.bfloat16, B=4, QN=2, KVN=2, Dqk=24, Dv=16,
                      sparse_mode=3, lq=L, lkv=L, seed=30)
    out, lse = assert_matches_reference(case)
    starts = np.concatenate([[0], np.cumsum(L)[:-1]])
    for b in range(4):
        sl = slice(starts[b], starts[b] + L[b])
        sub = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=1, QN=2, Sq=L[b], Dqk=24, Dv=16,
                         sparse_mode=3, seed=0)
        sub.q = case.q[sl].permute(1, 0, 2).unsqueeze(0).contiguous()
        sub.k = case.k[sl].permute(1, 0, 2).unsqueeze(0).contiguous()
        sub.v = case.v[sl].permute(1, 0, 2).unsqueeze(0).contiguous()
        so, sl_ = oracle.attention(sub)
        np.testing.assert_array_equal(out[sl].transpose(1, 0, 2), so[0])
        np.testing.assert_array_equal(lse[sl].T, sl_[0])


def test_bsnd_equals_bnsd_after_transpose():
    a = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=4, KVN=2, Sq=10, Dqk=16,
                   sparse_mode=3, lq=[10, 4], lkv=[10, 8], seed=31)
    b = W.make_fia(layout="BSND", dtype=torch.bfloat16, B=2, QN=4, KVN=2, Sq=10, Dqk=16,
                   sparse_mode=3, lq=[10, 4], lkv=[10, 8], seed=0)
    b.q = a.q.transpose(1, 2).contiguous()
    b.k = a.k.transpose(1, 2).contiguous()
    b.v = a.v.transpose(1, 2).contiguous()
    oa, la = oracle.attention(a)
    ob, lb = oracle.attention(b)
    np.testing.assert_array_equal(oa, ob.transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(la, lb)


def test_gqa_equals_explicit_kv_head_replication():
    a = W.make_fia(layout="BNSD", dtype=torch.float16, B=1, QN=6, KVN=2, Sq=9, Dqk=16,
                   sparse_mode=3, seed=32)
    r = W.make_fia(layout="BNSD", dtype=torch.float16, B=1, QN=6, KVN=6, Sq=9, Dqk=16,
                   sparse_mode=3, seed=0)
    r.q = a.q
    r.k = a.k.repeat_interleave(3, dim=1).contiguous()
    r.v = a.v.repeat_interleave(3, dim=1).contiguous()
    oa, la = oracle.attention(a)
    orr, lr = oracle.attention(r)
    np.testing.assert_array_equal(oa, orr)
    np.testing.assert_array_equal(la, lr)


# ---------------------------------------------------------------------------
# mask-mode invariants and the pages' empty-row conditions
# ---------------------------------------------------------------------------

def _pair(mode_a, mode_b, **kw):
    seed = kw.pop("seed")
    a = W.make_fia(sparse_mode=mode_a, seed=seed, **kw)
    b = W.make_fia(sparse_mode=mode_b, seed=seed, **kw)
    return a, b


def test_mode2_equals_mode3_when_lengths_match():
    a, b = _pair(2, 3, layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=14, Dqk=8,
                 lq=[14, 9], lkv=[14, 9], seed=40)
    np.testing.assert_array_equal(oracle.attention(a)[0], oracle.attention(b)[0])


def test_mode3_equals_mode1_with_rule_built_mask():
    a = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=10, Skv=16, Dqk=8,
                   lq=[10, 7], lkv=[16, 12], sparse_mode=3, seed=41)
    lq, lkv = a.lq, a.lkv
    b = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=10, Skv=16, Dqk=8,
                   lq=[10, 7], lkv=[16, 12], sparse_mode=1, seed=41,
                   mask_kind=lambda bb, i, j: j > i + (lkv[bb] - lq[bb]))
    oa, la = oracle.attention(a)
    ob, lb = oracle.attention(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_mode0_zero_mask_with_next0_equals_mode2():
    a, _ = _pair(0, 0, layout="BSND", dtype=torch.float16, B=1, QN=2, Sq=12, Dqk=8, seed=42,
                 pre_tokens=INT_MAX, next_tokens=0, mask_kind="zeros")
    b = W.make_fia(layout="BSND", dtype=torch.float16, B=1, QN=2, Sq=12, Dqk=8, seed=42,
                   sparse_mode=2)
    np.testing.assert_array_equal(oracle.attention(a)[0], oracle.attention(b)[0])


def test_mode4_open_band_equals_mode3():
    kw = dict(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=9, Skv=13, Dqk=8,
              lq=[9, 6], lkv=[13, 11], seed=43)
    a = W.make_fia(sparse_mode=4, pre_tokens=INT_MAX, next_tokens=0, **kw)
    b = W.make_fia(sparse_mode=3, **kw)
    np.testing.assert_array_equal(oracle.attention(a)[0], oracle.attention(b)[0])


@pytest.mark.parametrize("trial", range(40))
def test_empty_rows_exactly_where_the_pages_say(trial):
    # The interception conditions of the constraints (output-quant rows that
    # take part in no computation), under the band validity rule the TND
    # constraints state for mode 4 (pre + next >= 0).
    rng = np.random.default_rng(500 + trial)
    Lq, Lkv = int(rng.integers(2, 12)), int(rng.integers(1, 12))   # Q_S = 1 ignores pre/next
    pre = int(rng.integers(-4, 8))
    nxt = int(rng.integers(max(-6, -pre), 8))
    assert pre + nxt >= 0
    for mode in (0, 3, 4):
        case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=1, QN=1, Sq=Lq, Skv=Lkv,
                          Dqk=8, sparse_mode=mode, pre_tokens=pre, next_tokens=nxt,
                          mask_kind="zeros" if mode == 0 else None, seed=trial)
        _, lse = oracle.attention(case)
        any_empty = bool(np.isinf(lse).any())
        if mode == 0:
            cond = (Lq - Lkv - pre > 0) or (nxt < 0)
        elif mode == 3:
            cond = Lkv - Lq < 0
        else:
            cond = (pre < 0) or (nxt + Lkv - Lq < 0)
        assert any_empty == cond, (mode, Lq, Lkv, pre, nxt)


# ---------------------------------------------------------------------------
# decode and paged KV
# ---------------------------------------------------------------------------

def test_decode_equals_last_prefill_row():
    L = [17, 5, 30]
    pre = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=30, Dqk=16,
                     sparse_mode=3, lq=L, lkv=L, seed=50)
    op, lp = oracle.attention(pre)
    dec = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=1, Skv=30,
                     Dqk=16, lkv=L, seed=0)
    dec.q = torch.stack([pre.q[b, :, L[b] - 1:L[b]] for b in range(3)]).contiguous()
    dec.k, dec.v = pre.k, pre.v
    od, ld = oracle.attention(dec)
    for b in range(3):
        np.testing.assert_array_equal(od[b, :, 0], op[b, :, L[b] - 1])
        np.testing.assert_array_equal(ld[b, :, 0], lp[b, :, L[b] - 1])


@pytest.mark.parametrize("pool_layout", [0, 1])
def test_paged_equals_contiguous_after_gather(pool_layout):
    case = W.make_paged_decode(B=3, QN=4, KVN=2, D=16, lkv=[40, 3, 64], block_size=16,
                               pool_layout=pool_layout, seed=51, extra_blocks=2)
    out, lse = oracle.attention(case)
    bt = case.block_table.numpy()
    kp, vp = case.k, case.v
    if pool_layout == 1:
        kp = kp.reshape(kp.shape[0], 16, 2, 16).permute(0, 2, 1, 3)
        vp = vp.reshape(vp.shape[0], 16, 2, 16).permute(0, 2, 1, 3)
    S = bt.shape[1] * 16
    kc = torch.zeros(3, 2, S, 16, dtype=kp.dtype)
    vc = torch.zeros(3, 2, S, 16, dtype=vp.dtype)
    for b in range(3):
        for c in range(bt.shape[1]):
            if bt[b, c] >= 0:
                kc[b, :, c * 16:(c + 1) * 16] = kp[bt[b, c]]
                vc[b, :, c * 16:(c + 1) * 16] = vp[bt[b, c]]
    cont = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=1, Skv=S,
                      Dqk=16, lkv=case.lkv, seed=0)
    cont.q, cont.k, cont.v = case.q, kc, vc
    oc, lc = oracle.attention(cont)
    np.testing.assert_array_equal(out, oc)
    np.testing.assert_array_equal(lse, lc)


def _gather_pool(case):
    """Contiguous BNSD copies [B, KVN, cols * bs, D] of a paged pool (rows of
    unused table entries stay zero)."""
    bt = case.block_table.numpy()
    bs, KVN, D = case.block_size, case.KVN, case.Dqk
    kp, vp = case.k, case.v
    if case.pool_layout == 1:
        kp = kp.reshape(kp.shape[0], bs, KVN, D).permute(0, 2, 1, 3)
        vp = vp.reshape(vp.shape[0], bs, KVN, D).permute(0, 2, 1, 3)
    S = bt.shape[1] * bs
    kc = torch.zeros(case.B, KVN, S, D, dtype=kp.dtype)
    vc = torch.zeros(case.B, KVN, S, D, dtype=vp.dtype)
    for b in range(case.B):
        for c in range(bt.shape[1]):
            if bt[b, c] >= 0:
                kc[b, :, c * bs:(c + 1) * bs] = kp[bt[b, c]]
                vc[b, :, c * bs:(c + 1) * bs] = vp[bt[b, c]]
    return kc, vc


@pytest.mark.parametrize("pool_layout", [0, 1])
@pytest.mark.parametrize("mode", [0, 3, 4])
def test_tnd_paged_prefill_equals_contiguous_tnd_after_gather(pool_layout, mode):
    # TND query with a paged cache (v2 page, TND constraints: page attention
    # with block size 128 / 512 / 1024, cumulative actual_seq_kvlen): equals
    # the contiguous TND oracle on the pool gathered batch by batch and
    # concatenated, bit for bit
    lq, lkv = [70, 1, 130], [200, 1, 300]
    mk = "template" if mode in (3, 4) else None
    case = W.make_paged_prefill(layout="TND", B=3, QN=4, KVN=2, D=16, lq=lq, lkv=lkv,
                                block_size=128, pool_layout=pool_layout, sparse_mode=mode,
                                pre_tokens=50, next_tokens=20, mask_kind=mk, extra_blocks=2,
                                seed=95 + mode + 4 * pool_layout)
    assert list(case.seq_kvlen_arg()) == list(np.cumsum(lkv))
    out, lse = oracle.attention(case)
    kc, vc = _gather_pool(case)                     # [B, KVN, cols * bs, D]
    kt = torch.cat([kc[b, :, :lkv[b]].permute(1, 0, 2) for b in range(3)])   # [T_kv, KVN, D]
    vt = torch.cat([vc[b, :, :lkv[b]].permute(1, 0, 2) for b in range(3)])
    cont = W.make_fia(layout="TND", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Dqk=16, lq=lq, lkv=lkv,
                      sparse_mode=mode, pre_tokens=50, next_tokens=20, mask_kind=mk, seed=0)
    cont.q, cont.k, cont.v = case.q, kt.contiguous(), vt.contiguous()
    oc, lc = oracle.attention(cont)
    np.testing.assert_array_equal(out, oc)
    np.testing.assert_array_equal(lse, lc)
    # and per-sequence runs: each sequence's rows equal a BNSD run of its own
    start = 0
    for b in range(3):
        one = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=1, QN=4, KVN=2, Sq=lq[b], Skv=lkv[b],
                         Dqk=16, sparse_mode=mode, pre_tokens=50, next_tokens=20, mask_kind=mk, seed=0)
        one.q = case.q[start:start + lq[b]].permute(1, 0, 2).unsqueeze(0).contiguous()
        one.k = kc[b:b + 1, :, :lkv[b]].contiguous()
        one.v = vc[b:b + 1, :, :lkv[b]].contiguous()
        o1, l1 = oracle.attention(one)
        np.testing.assert_array_equal(out[start:start + lq[b]], o1[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(lse[start:start + lq[b]], l1[0].T)
        start += lq[b]


@pytest.mark.parametrize("pool_layout", [0, 1])
@pytest.mark.parametrize("mode", [0, 3, 4])
def test_paged_prefill_equals_contiguous_after_gather(pool_layout, mode):
    # chunked prefill: query chunks shorter than the cached kv
    case = W.make_paged_prefill(layout="BNSD", B=3, QN=4, KVN=2, D=16, Sq=12, lq=[12, 5, 9],
                                lkv=[40, 5, 130], block_size=32, pool_layout=pool_layout,
                                sparse_mode=mode, pre_tokens=20, next_tokens=3, seed=56,
                                extra_blocks=3)
    out, lse = oracle.attention(case)
    kc, vc = _gather_pool(case)
    cont = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=12,
                      Skv=kc.shape[2], Dqk=16, lq=case.lq, lkv=case.lkv, sparse_mode=mode,
                      pre_tokens=20, next_tokens=3, seed=0)
    cont.q, cont.k, cont.v = case.q, kc, vc
    oc, lc = oracle.attention(cont)
    np.testing.assert_array_equal(out, oc)
    np.testing.assert_array_equal(lse, lc)


def test_multi_token_decode_equals_last_rows_of_causal_prefill():
    # sparse_mode 3 aligns the query rows bottom-right: the Q_S query tokens
    # of a decode step see what the last Q_S rows of a full causal prefill see
    L, QS = [37, 9, 64], 4
    full = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=64, Dqk=16,
                      sparse_mode=3, lq=L, lkv=L, seed=57)
    of, lf = oracle.attention(full)
    mtp = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=QS, Skv=64,
                     Dqk=16, sparse_mode=3, lkv=L, seed=0)
    mtp.q = torch.stack([full.q[b, :, L[b] - QS:L[b]] for b in range(3)]).contiguous()
    mtp.k, mtp.v = full.k, full.v
    om, lm = oracle.attention(mtp)
    for b in range(3):
        np.testing.assert_array_equal(om[b], of[b, :, L[b] - QS:L[b]])
        np.testing.assert_array_equal(lm[b], lf[b, :, L[b] - QS:L[b]])
    # the first query token of the step sees every key but the last QS - 1
    assert np.all(np.isfinite(lm))


def test_decode_mask_equals_decode_over_the_kept_keys():
    # query S == 1 with a per-(batch, kv token) mask: the same as decoding
    # against only the unmasked keys, gathered into a shorter cache
    case = W.make_fia(layout="BSND", dtype=torch.bfloat16, B=3, QN=4, KVN=2, Sq=1, Skv=50,
                      Dqk=16, lkv=[50, 7, 33], mask_kind="random", seed=58)
    out, lse = oracle.attention(case)
    m = case.atten_mask.numpy().reshape(3, -1)
    for b in range(3):
        keep = np.nonzero(m[b, :int(case.lkv[b])] == 0)[0]
        sub = W.make_fia(layout="BSND", dtype=torch.bfloat16, B=1, QN=4, KVN=2, Sq=1,
                         Skv=max(len(keep), 1), Dqk=16, lkv=[len(keep)], seed=0)
        sub.q = case.q[b:b + 1]
        if len(keep):
            sub.k = case.k[b:b + 1, torch.from_numpy(keep)].contiguous()
            sub.v = case.v[b:b + 1, torch.from_numpy(keep)].contiguous()
        else:
            sub.k = case.k[b:b + 1, :1].contiguous()
            sub.v = case.v[b:b + 1, :1].contiguous()
        os_, ls_ = oracle.attention(sub)
        np.testing.assert_array_equal(out[b], os_[0])
        np.testing.assert_array_equal(lse[b], ls_[0])


def test_decode_mask_fully_masked_batch_and_broadcast():
    case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=1, Skv=20, Dqk=8,
                      seed=59)
    m = np.zeros((2, 20), dtype=np.uint8)
    m[1] = 1                                   # batch 1: every key masked
    m[0, 5:9] = 1
    case.atten_mask = torch.from_numpy(m)
    out, lse = oracle.attention(case)
    assert np.all(out[1] == 0) and np.all(np.isposinf(lse[1]))
    assert np.all(np.isfinite(lse[0]))
    # a leading 1 broadcasts over the batch
    case.atten_mask = torch.from_numpy(m[:1].copy())
    ob, lb = oracle.attention(case)
    np.testing.assert_array_equal(ob[0], out[0])
    case.atten_mask = torch.from_numpy(np.repeat(m[:1], 2, axis=0))
    orep, lrep = oracle.attention(case)
    np.testing.assert_array_equal(ob, orep)
    np.testing.assert_array_equal(lb, lrep)


def test_row_subset_matches_full_run():
    case = W.make_fia(layout="BSND", dtype=torch.bfloat16, B=2, QN=4, KVN=2, Sq=20, Dqk=16,
                      sparse_mode=3, lq=[20, 13], lkv=[20, 13], seed=52)
    out, lse = oracle.attention(case)
    rows = [(0, 1, 5), (1, 3, 12), (1, 0, 0), (0, 2, 19), (1, 2, 17)]
    so, sl = oracle.attention(case, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(so[r], out[b, i, h])
        assert sl[r] == lse[b, h, i]


def test_padding_rows_are_zero_and_plus_inf():
    case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=8, Dqk=8,
                      sparse_mode=3, lq=[8, 3], lkv=[8, 3], seed=53, nan_padding=True)
    out, lse = oracle.attention(case)
    assert np.all(out[1, :, 3:] == 0) and np.all(np.isposinf(lse[1, :, 3:]))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse[0]))


def test_empty_kv_gives_zero_and_plus_inf():
    case = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=1, Skv=8, Dqk=8,
                      lkv=[0, 5], seed=54)
    out, lse = oracle.attention(case)
    assert np.all(out[0] == 0) and np.all(np.isposinf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------------------
# block-sparse
# ---------------------------------------------------------------------------

def _bsa_as_fia(bc, mode, mask_fn=None):
    f = W.make_fia(layout=bc.layout, dtype=bc.dtype, B=bc.B, QN=bc.QN, KVN=bc.KVN, Sq=bc.Sq,
                   Skv=bc.Skv, Dqk=bc.D, lq=bc.lq, lkv=bc.lkv, scale=bc.scale, sparse_mode=mode,
                   mask_kind=mask_fn, seed=0)
    f.q, f.k, f.v = bc.q, bc.k, bc.v
    return f


def test_bsa_all_ones_equals_dense():
    bc = W.make_bsa(layout="BNSD", B=2, QN=4, KVN=2, Sq=40, Skv=56, D=16, X=16, Y=16,
                    lq=[40, 29], lkv=[56, 33], mask_kind="ones", seed=60)
    ob, lb = oracle.block_sparse(bc)
    od, ld = oracle.attention(_bsa_as_fia(bc, 0))
    np.testing.assert_array_equal(ob, od)
    np.testing.assert_array_equal(lb, ld)


def test_bsa_diagonal_equals_chunked_dense():
    bc = W.make_bsa(layout="BNSD", B=1, QN=2, KVN=1, Sq=48, D=16, X=16, Y=16,
                    mask_kind="diag", seed=61)
    ob, lb = oracle.block_sparse(bc)
    for c in range(3):
        f = W.make_fia(layout="BNSD", dtype=bc.dtype, B=1, QN=2, KVN=1, Sq=16, Dqk=16,
                       scale=bc.scale, seed=0)
        sl = slice(16 * c, 16 * (c + 1))
        f.q, f.k, f.v = (t[:, :, sl].contiguous() for t in (bc.q, bc.k, bc.v))
        od, ld = oracle.attention(f)
        np.testing.assert_array_equal(ob[:, :, sl], od)
        np.testing.assert_array_equal(lb[:, :, sl], ld)


def test_bsa_block_lower_triangular_equals_mode1_block_causal_mask():
    bc = W.make_bsa(layout="BSND", B=1, QN=2, KVN=2, Sq=48, D=16, X=16, Y=16,
                    mask_kind="lower", seed=62)
    ob, lb = oracle.block_sparse(bc)
    od, ld = oracle.attention(_bsa_as_fia(bc, 1, lambda b, i, j: j // 16 > i // 16))
    np.testing.assert_array_equal(ob, od)
    np.testing.assert_array_equal(lb, ld)


def test_bsa_matches_torch_reference_with_ragged_lengths():
    bc = W.make_bsa(layout="TND", B=2, QN=4, KVN=2, D=16, X=8, Y=16, lq=[21, 9],
                    lkv=[37, 12], p=0.4, seed=63)
    ob, lb = oracle.block_sparse(bc)
    m = bc.block_mask.numpy()
    for b in range(2):
        Lq, Lkv = int(bc.lq[b]), int(bc.lkv[b])
        q0, k0 = int(bc.lq[:b].sum()), int(bc.lkv[:b].sum())
        q = bc.q[q0:q0 + Lq].to(torch.float64).permute(1, 0, 2)
        k = bc.k[k0:k0 + Lkv].to(torch.float64).permute(1, 0, 2).repeat_interleave(2, 0)
        v = bc.v[k0:k0 + Lkv].to(torch.float64).permute(1, 0, 2).repeat_interleave(2, 0)
        keep = torch.from_numpy(np.kron(m[b], np.ones((8, 16), dtype=np.uint8))[:, :Lq, :Lkv] != 0)
        s = bc.scale * torch.matmul(q, k.transpose(1, 2))
        s = s.masked_fill(~keep, float("-inf"))
        ref = torch.nan_to_num(torch.softmax(s, -1), nan=0.0) @ v
        lse = torch.logsumexp(s, -1)
        empty = ~keep.any(-1)
        ref[empty] = 0
        lse[empty] = float("inf")
        np.testing.assert_allclose(ob[q0:q0 + Lq].transpose(1, 0, 2), ref.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(lb[q0:q0 + Lq].T, lse.numpy(), atol=1e-11, rtol=0)


def test_bsa_compaction_brute_force():
    rng = np.random.default_rng(64)
    m = (rng.random((2, 3, 5, 7)) < 0.5).astype(np.uint8)
    lq, lkv, X, Y = [70, 33], [100, 45], 16, 16
    idx, cnt = oracle.bsa_compact(m, lq, lkv, X, Y)
    for b in range(2):
        for h in range(3):
            for qb in range(5):
                sel = []
                if qb * X < lq[b]:
                    sel = [kb for kb in range(7) if m[b, h, qb, kb] and kb * Y < lkv[b]]
                assert cnt[b, h, qb] == len(sel)
                assert list(idx[b, h, qb]) == sel + [-1] * (7 - len(sel))


def test_workload_generator_is_deterministic():
    a = W.c1_dense_causal_fp16()
    b = W.c1_dense_causal_fp16()
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert list(W.c2_lengths()) == list(W.c2_lengths())
    assert W.c4_lengths().min() >= 64 and W.c4_lengths().max() <= 8192


# ---------------------------------------------------------------------------
# KV pseudo-quantization (int8 key/value, value = scale * (x + offset))
# ---------------------------------------------------------------------------

def _dequantized(case):
    """bf16 copy of an int8 case with the dequantized cache, built with
    torch ops from the same reading; exact when the values fit bf16."""
    qt = case.quant
    B, KVN, D = case.B, case.KVN, case.Dqk

    def deq(x, mode, sc, of):
        xb = x.to(torch.float64)
        if case.layout == "BNSD":
            xb = xb                                   # [B, KVN, S, D]
        else:
            xb = xb.permute(0, 2, 1, 3)               # BSND -> [B, KVN, S, D]
        if mode == 0:
            s = sc.to(torch.float64).reshape(1, KVN, 1, D)
            o = of.to(torch.float64).reshape(1, KVN, 1, D) if of is not None else 0.0
        else:
            S = xb.shape[2]
            s = sc.to(torch.float64)[:, :S].reshape(B, 1, S, 1)
            o = of.to(torch.float64)[:, :S].reshape(B, 1, S, 1) if of is not None else 0.0
        y = s * (xb + o)
        if case.layout != "BNSD":
            y = y.permute(0, 2, 1, 3)
        yb = y.to(torch.bfloat16)
        assert torch.equal(yb.to(torch.float64), y), "dequantized cache not exact in bf16"
        return yb.contiguous()

    k = deq(case.k, qt["key_quant_mode"], qt["dequant_scale_key"], qt["dequant_offset_key"])
    v = deq(case.v, qt["value_quant_mode"], qt["dequant_scale_value"], qt["dequant_offset_value"])
    ref = W.make_fia(layout=case.layout, dtype=torch.bfloat16, B=B, QN=case.QN, KVN=KVN,
                     Sq=case.Sq, Skv=case.Skv, Dqk=D, lkv=case.lkv, sparse_mode=case.sparse_mode,
                     seed=0)
    ref.q, ref.k, ref.v = case.q, k, v
    return ref


@pytest.mark.parametrize("kmode, vmode", [(0, 0), (1, 1), (0, 1), (1, 0)])
@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
def test_int8_kv_equals_bf16_on_the_dequantized_cache(kmode, vmode, layout):
    # power-of-two scales and integer offsets: the dequantized cache is exact
    # in bf16, so the int8 oracle must equal the bf16 oracle on it exactly
    case = W.make_quant_decode(layout=layout, B=3, QN=4, KVN=2, D=16, lkv=[40, 3, 17],
                               kmode=kmode, vmode=vmode, pow2=True, seed=70 + 2 * kmode + vmode)
    out, lse = oracle.attention(case)
    ro, rl = oracle.attention(_dequantized(case))
    np.testing.assert_array_equal(out, ro)
    np.testing.assert_array_equal(lse, rl)


def test_int8_kv_unit_scale_is_the_raw_integers():
    case = W.make_quant_decode(layout="BNSD", B=2, QN=2, KVN=1, D=8, lkv=[9, 4], kmode=1, vmode=0,
                               unit=True, seed=75)
    out, lse = oracle.attention(case)
    ref = W.make_fia(layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, KVN=1, Sq=1, Skv=9, Dqk=8,
                     lkv=[9, 4], seed=0)
    ref.q, ref.k, ref.v = case.q, case.k.to(torch.bfloat16), case.v.to(torch.bfloat16)
    ro, rl = oracle.attention(ref)
    np.testing.assert_array_equal(out, ro)
    np.testing.assert_array_equal(lse, rl)


@pytest.mark.parametrize("pool_layout", [0, 1])
@pytest.mark.parametrize("kmode, vmode", [(0, 0), (1, 1), (0, 1)])
def test_paged_int8_kv_equals_contiguous_after_gather(pool_layout, kmode, vmode):
    # page attention with an int8 cache (v2 page, query S 1 page attention
    # scenario: int8 key/value allowed): the paged oracle equals the
    # contiguous int8 oracle on the gathered pool, with the same per-channel
    # or per-token (logical kv position) scales and offsets, bit for bit
    case = W.make_quant_decode(layout="BNSD", B=3, QN=4, KVN=2, D=16, lkv=[70, 5, 64],
                               kmode=kmode, vmode=vmode, block_size=32, pool_layout=pool_layout,
                               extra_blocks=2, seed=80 + 2 * kmode + vmode + 4 * pool_layout)
    out, lse = oracle.attention(case)
    kc, vc = _gather_pool(case)
    cont = W.make_quant_decode(layout="BNSD", B=3, QN=4, KVN=2, D=16, lkv=[70, 5, 64],
                               Skv=kc.shape[2], kmode=kmode, vmode=vmode, seed=0)
    cont.q, cont.k, cont.v = case.q, kc, vc
    cont.quant = dict(case.quant)
    oc, lc = oracle.attention(cont)
    np.testing.assert_array_equal(out, oc)
    np.testing.assert_array_equal(lse, lc)
    # and with power-of-two scales, the bf16 oracle on the dequantized pool
    case2 = W.make_quant_decode(layout="BNSD", B=3, QN=4, KVN=2, D=16, lkv=[70, 5, 64],
                                kmode=kmode, vmode=vmode, block_size=32, pool_layout=pool_layout,
                                pow2=True, seed=90 + 2 * kmode + vmode + 4 * pool_layout)
    kc2, vc2 = _gather_pool(case2)
    cont2 = W.make_quant_decode(layout="BNSD", B=3, QN=4, KVN=2, D=16, lkv=[70, 5, 64],
                                Skv=kc2.shape[2], kmode=kmode, vmode=vmode, seed=0)
    cont2.q, cont2.k, cont2.v = case2.q, kc2, vc2
    cont2.quant = dict(case2.quant)
    out2, lse2 = oracle.attention(case2)
    ro, rl = oracle.attention(_dequantized(cont2))
    np.testing.assert_array_equal(out2, ro)
    np.testing.assert_array_equal(lse2, rl)


def test_int8_kv_multi_token_causal():
    case = W.make_quant_decode(layout="BNSD", B=2, QN=4, KVN=2, D=16, Sq=3, lkv=[20, 2],
                               kmode=0, vmode=1, pow2=True, sparse_mode=3, seed=76)
    out, lse = oracle.attention(case)
    ro, rl = oracle.attention(_dequantized(case))
    np.testing.assert_array_equal(out, ro)
    np.testing.assert_array_equal(lse, rl)


# ---------------------------------------------------------------------------
# block-sparse FP8 (E4M3FN values times per-block fp32 scales)
# ---------------------------------------------------------------------------

def test_e4m3fn_reader_matches_library_cast():
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.read_e4m3fn(int(b)) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def _bsa_fp8_as_bf16(case):
    """The same case with bf16 inputs holding the dequantized values (exact
    when the per-block scales are powers of two)."""
    def deq(x, sc, blk):
        xb = x.to(torch.float64)
        if case.layout != "BNSD":
            xb = xb.permute(0, 2, 1, 3)
        S = xb.shape[2]
        rep = sc.to(torch.float64)[..., 0].repeat_interleave(blk, dim=2)[:, :, :S]
        y = xb * rep[..., None]
        if case.layout != "BNSD":
            y = y.permute(0, 2, 1, 3)
        yb = y.to(torch.bfloat16)
        assert torch.equal(yb.to(torch.float64), y)
        return yb.contiguous()

    f = case.fp8
    ref = W.make_bsa(layout=case.layout, B=case.B, QN=case.QN, KVN=case.KVN, Sq=case.Sq,
                     Skv=case.Skv, D=case.D, X=case.X, Y=case.Y, lq=case.lq, lkv=case.lkv,
                     scale=case.scale, mask_kind=case.block_mask.numpy(), seed=0)
    ref.q = deq(case.q, f["dequant_scale_query"], case.X)
    ref.k = deq(case.k, f["dequant_scale_key"], case.Y)
    ref.v = deq(case.v, f["dequant_scale_value"], case.Y)
    return ref


@pytest.mark.parametrize("layout, Y", [("BNSD", 256), ("BSND", 512)])
def test_bsa_fp8_equals_bf16_on_the_dequantized_inputs(layout, Y):
    case = W.make_bsa_fp8(layout=layout, B=2, QN=4, KVN=2, Sq=300, Skv=700, D=16, Y=Y, p=0.5,
                          lq=[300, 129], lkv=[700, 260], pow2=True, seed=80)
    out, lse = oracle.block_sparse(case)
    ro, rl = oracle.block_sparse(_bsa_fp8_as_bf16(case))
    np.testing.assert_array_equal(out, ro)
    np.testing.assert_array_equal(lse, rl)


def _gather_rows(pool, bt, bs, pool_layout):
    """[B, cols * bs, d] float64 copy of a single-kv-head paged pool."""
    p = pool.to(torch.float64).numpy()
    if pool_layout == 0:
        p = p[:, 0]
    out = np.zeros((bt.shape[0], bt.shape[1] * bs, p.shape[-1]))
    for b in range(bt.shape[0]):
        for c in range(bt.shape[1]):
            if bt[b, c] >= 0:
                out[b, c * bs:(c + 1) * bs] = p[bt[b, c]]
    return out


@pytest.mark.parametrize("pool_layout", [0, 1])
@pytest.mark.parametrize("layout,S", [("BSND", 1), ("BNSD", 3), ("BSH", 2)])
def test_mla_equals_brute_force_on_concatenated_vectors(pool_layout, layout, S):
    # MLA (query_rope / key_rope): the score is scale * (q.k + q_rope.k_rope),
    # i.e. attention over the concatenated [q, q_rope] and [k, k_rope] vectors,
    # with value and output keeping D; query S > 1 is bottom-right causal
    case = W.make_mla_decode(layout=layout, B=3, QN=4, Sq=S, lkv=[37, 5, 64], block_size=16,
                             D=24, Dr=8, pool_layout=pool_layout, seed=61, extra_blocks=2)
    out, lse = oracle.attention(case)
    bt = case.block_table.numpy()
    K = _gather_rows(case.k, bt, 16, pool_layout)
    KR = _gather_rows(case.rope["key_rope"], bt, 16, pool_layout)
    V = _gather_rows(case.v, bt, 16, pool_layout)

    def bnsd(t, d):
        x = t.to(torch.float64)
        if layout == "BSH":
            x = x.reshape(case.B, S, case.QN, d)
        if layout != "BNSD":
            x = x.permute(0, 2, 1, 3)
        return x.numpy()

    q, qr = bnsd(case.q, 24), bnsd(case.rope["query_rope"], 8)
    o = out if layout == "BNSD" else np.transpose(out, (0, 2, 1, 3))
    for b in range(case.B):
        L = int(case.lkv[b])
        for h in range(case.QN):
            for t in range(S):
                n = L - S + t + 1 if S > 1 else L       # keys j <= L - S + t
                s = case.scale * (K[b, :n] @ q[b, h, t] + KR[b, :n] @ qr[b, h, t])
                w = np.exp(s - s.max())
                assert np.max(np.abs(o[b, h, t] - w @ V[b, :n] / w.sum())) < 1e-12
                assert abs(lse[b, h, t] - (s.max() + math.log(w.sum()))) < 1e-12


def test_mla_zero_key_rope_equals_plain_attention():
    case = W.make_mla_decode(B=2, QN=8, Sq=1, lkv=[50, 17], block_size=16, D=32, Dr=8, seed=62)
    case.rope["key_rope"] = torch.zeros_like(case.rope["key_rope"])
    out, lse = oracle.attention(case)
    case.rope = None
    out0, lse0 = oracle.attention(case)
    assert np.array_equal(out, out0) and np.array_equal(lse, lse0)


@pytest.mark.parametrize("mode_causal", [True, False])
def test_mla_tnd_equals_brute_force(mode_causal):
    # TND MLA decode: batch b's lq_b query tokens are rows q_start_b .. of
    # the (T, N, D) query; kv lengths are per batch with the paged cache
    lq = [1, 3, 4] if mode_causal else [1, 1, 1]
    case = W.make_mla_decode(layout="TND", B=3, QN=4, lq=lq, lkv=[37, 2, 64], block_size=16,
                             D=24, Dr=8, pool_layout=1, seed=63, extra_blocks=1)
    assert case.sparse_mode == (3 if mode_causal else 0)
    out, lse = oracle.attention(case)
    bt = case.block_table.numpy()
    K = _gather_rows(case.k, bt, 16, 1)
    KR = _gather_rows(case.rope["key_rope"], bt, 16, 1)
    V = _gather_rows(case.v, bt, 16, 1)
    q = case.q.to(torch.float64).numpy()
    qr = case.rope["query_rope"].to(torch.float64).numpy()
    row = 0
    for b in range(3):
        L = int(case.lkv[b])
        for t in range(lq[b]):
            n = L - lq[b] + t + 1 if mode_causal else L
            for h in range(4):
                if n <= 0:
                    assert np.all(out[row, h] == 0) and np.isposinf(lse[row, h])
                    continue
                s = case.scale * (K[b, :n] @ q[row, h] + KR[b, :n] @ qr[row, h])
                w = np.exp(s - s.max())
                assert np.max(np.abs(out[row, h] - w @ V[b, :n] / w.sum())) < 1e-12
                assert abs(lse[row, h] - (s.max() + math.log(w.sum()))) < 1e-12
            row += 1


@pytest.mark.parametrize("S,pre,nxt", [(1, 20, 0), (1, 5, 3), (3, 7, 0), (4, 10, 2), (2, 0, 0)])
@pytest.mark.parametrize("pool_layout", [0, 1])
def test_mla_band_equals_brute_force(S, pre, nxt, pool_layout):
    # MLA with sparse_mode 4: query token t of batch b sees the keys
    # Lkv - S + t - pre <= j <= Lkv - S + t + next, at query S 1 too
    case = W.make_mla_decode(layout="BSND", B=3, QN=4, Sq=S, lkv=[37, 2, 64], block_size=16,
                             D=24, Dr=8, pool_layout=pool_layout, seed=64, extra_blocks=1,
                             band=(pre, nxt))
    assert case.sparse_mode == 4
    out, lse = oracle.attention(case)
    bt = case.block_table.numpy()
    K = _gather_rows(case.k, bt, 16, pool_layout)
    KR = _gather_rows(case.rope["key_rope"], bt, 16, pool_layout)
    V = _gather_rows(case.v, bt, 16, pool_layout)
    q = case.q.to(torch.float64).numpy()                        # [B, S, N, D]
    qr = case.rope["query_rope"].to(torch.float64).numpy()
    for b in range(3):
        L = int(case.lkv[b])
        for t in range(S):
            lo, hi = max(0, L - S + t - pre), min(L - 1, L - S + t + nxt)
            for h in range(4):
                if hi < lo:
                    assert np.all(out[b, t, h] == 0) and np.isposinf(lse[b, h, t])
                    continue
                s = case.scale * (K[b, lo:hi + 1] @ q[b, t, h] + KR[b, lo:hi + 1] @ qr[b, t, h])
                w = np.exp(s - s.max())
                assert np.max(np.abs(out[b, t, h] - w @ V[b, lo:hi + 1] / w.sum())) < 1e-12
                assert abs(lse[b, h, t] - (s.max() + math.log(w.sum()))) < 1e-12
