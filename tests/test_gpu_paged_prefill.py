"""GPU parity of prefill and multi-token decode (query S > 1) against a paged
KV cache: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs.  The oracle reads key/value token j of batch b at row
j % block_size of pool block block_table[b][j / block_size] (page attention
scenario of the fused-infer-attention pages); the pool's unreferenced blocks
and the rows past each batch's length in its last block hold NaN, so any read
outside the table's valid entries would show up in the output."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import (compare, compare_rows, fia_plan, head_rows, run, say, seeded_subset, to_dev,
                     TOL_LSE, TOL_OUT)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check(case):
    say(f"[paged] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"Sq={case.Sq} lq={None if case.lq is None else list(case.lq)} lkv={list(case.lkv)} "
        f"D={case.Dqk} bs={case.block_size} pool={case.pool_layout} mode={case.sparse_mode} "
        f"dtype={case.dtype}")
    ref_out, ref_lse = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err = compare(case, out, lse, ref_out, ref_lse)
    plan.close()
    return err


@pytest.mark.parametrize("pool_layout", [0, 1])
@pytest.mark.parametrize("mode", [0, 2, 3, 4])
def test_paged_prefill_modes(pool_layout, mode):
    # chunked prefill: query chunks against longer cached kv; batch 2 spans
    # more than 64 blocks (the kernel's block-id window moves)
    case = W.make_paged_prefill(f"paged_m{mode}_p{pool_layout}", layout="BNSD", B=3, QN=8, KVN=2,
                                D=128, Sq=300, lq=[300, 77, 129], lkv=[700, 77, 8500],
                                block_size=128, pool_layout=pool_layout, sparse_mode=mode,
                                pre_tokens=300, next_tokens=40,
                                mask_kind="template" if mode >= 2 else None,
                                seed=300 + mode, extra_blocks=5, nan_pool=True)
    check(case)


TND_CASES = [
    # name, block_size, pool_layout, mode, D, QN, KVN, lq, lkv, dtype
    ("bs128_pl0_m3", 128, 0, 3, 128, 8, 2, [300, 1, 129, 77], [700, 1, 129, 2000], torch.bfloat16),
    ("bs512_pl1_m0", 512, 1, 0, 128, 4, 4, [64, 200], [5000, 200], torch.bfloat16),
    ("bs1024_pl0_m4", 1024, 0, 4, 128, 16, 4, [150, 90, 33], [3000, 90, 1500], torch.bfloat16),
    ("bs1024_pl1_m3_long", 1024, 1, 3, 64, 4, 1, [257, 1000], [70000, 1000], torch.float16),
    ("bs128_pl1_m3_f16", 128, 1, 3, 64, 2, 2, [5, 333], [5, 4096], torch.float16),
]


@pytest.mark.parametrize("case_args", TND_CASES, ids=[c[0] for c in TND_CASES])
def test_tnd_paged_prefill(case_args):
    # a TND query against a paged cache (TND constraints: block size 128,
    # 512 or 1024, cumulative actual_seq_kvlen); the 70000-token cache spans
    # more than 64 blocks of 1024 (the kernel's block-id window moves)
    name, bs, pl, mode, D, QN, KVN, lq, lkv, dtype = case_args
    case = W.make_paged_prefill(f"tnd_paged_{name}", layout="TND", dtype=dtype, B=len(lq), QN=QN,
                                KVN=KVN, D=D, lq=lq, lkv=lkv, block_size=bs, pool_layout=pl,
                                sparse_mode=mode, pre_tokens=120, next_tokens=30,
                                mask_kind="template" if mode >= 3 else None,
                                seed=340 + bs // 128 + mode, extra_blocks=2, nan_pool=True)
    check(case)


@pytest.mark.parametrize("layout, bs, dtype, D", [
    ("BSND", 256, torch.float16, 64),
    ("BSH", 384, torch.bfloat16, 128),
    ("BNSD", 512, torch.float16, 128),
])
def test_paged_prefill_layouts_block_sizes(layout, bs, dtype, D):
    case = W.make_paged_prefill(f"paged_{layout}_bs{bs}", layout=layout, dtype=dtype, B=3, QN=4,
                                KVN=1, D=D, Sq=200, lq=[200, 1, 64], lkv=[1000, 1, 64],
                                block_size=bs, pool_layout=1, sparse_mode=3,
                                mask_kind="template", seed=310 + bs, extra_blocks=2,
                                table_cols=9, nan_pool=True)
    check(case)


@pytest.mark.parametrize("mode", [0, 1])
def test_paged_prefill_explicit_mask(mode):
    case = W.make_paged_prefill(f"paged_mask_m{mode}", layout="BNSD", B=2, QN=4, KVN=2, D=128,
                                Sq=160, lq=[160, 90], lkv=[400, 90], block_size=128,
                                pool_layout=0, sparse_mode=mode, pre_tokens=250, next_tokens=10,
                                mask_kind="random", seed=320 + mode, nan_pool=True)
    check(case)


@pytest.mark.parametrize("QS", [2, 4, 16])
@pytest.mark.parametrize("G", [4, 8])
def test_multi_token_decode_paged(QS, G):
    # Q_S query tokens per sequence at the end of the cache (sparse_mode 3:
    # token t sees keys j <= Lkv - Q_S + t)
    case = W.make_paged_prefill(f"mtp{QS}_g{G}", layout="BNSD", B=4, QN=2 * G, KVN=2, D=128,
                                Sq=QS, lkv=[2000, QS, 129, 700], block_size=128, pool_layout=0,
                                sparse_mode=3, mask_kind="template", seed=330 + QS + G,
                                extra_blocks=1, nan_pool=True)
    check(case)


@pytest.mark.parametrize("layout, QS, G, mode, dtype, D", [
    ("BSND", 8, 2, 3, torch.bfloat16, 128),
    ("BNSD", 4, 4, 0, torch.bfloat16, 128),
    ("BSH", 2, 8, 3, torch.float16, 64),
    ("BNSD", 16, 1, 3, torch.float16, 128),
    ("BSND", 3, 5, 3, torch.bfloat16, 64),
])
def test_multi_token_decode_contiguous(layout, QS, G, mode, dtype, D):
    # contiguous KV, per-batch query lengths below S (padding rows) and one
    # batch with fewer keys than query tokens (rows without keys under mode 3)
    case = W.make_fia(f"mtp_{layout}_s{QS}_g{G}_m{mode}", layout=layout, dtype=dtype, B=4,
                      QN=2 * G, KVN=2, Sq=QS, Skv=1300, Dqk=D, sparse_mode=mode,
                      lq=[QS, max(QS - 1, 1), QS, 0], lkv=[1300, 77, QS - 1, 50],
                      mask_kind="template" if mode == 3 else None, seed=360 + QS + G,
                      nan_padding=True)
    say(f"[mtp] {case.name}")
    ref_out, ref_lse = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    compare(case, out, lse, ref_out, ref_lse)
    plan.close()


def test_multi_token_decode_equals_last_prefill_rows_on_gpu():
    L, QS = [900, 131], 4
    full = W.make_fia("mtp_vs_prefill", layout="BNSD", dtype=torch.bfloat16, B=2, QN=8, KVN=2,
                      Sq=900, Dqk=128, sparse_mode=3, lq=L, lkv=L, seed=340)
    mtp = W.make_fia("mtp_vs_prefill_q", layout="BNSD", dtype=torch.bfloat16, B=2, QN=8, KVN=2,
                     Sq=QS, Skv=900, Dqk=128, sparse_mode=3, lkv=L, seed=0)
    mtp.q = torch.stack([full.q[b, :, L[b] - QS:L[b]] for b in range(2)]).contiguous()
    mtp.k, mtp.v = full.k, full.v
    to_dev(full)
    to_dev(mtp)
    pf, pm = fia_plan(full), fia_plan(mtp)
    of, lf = run(pf)
    om, lm = run(pm)
    for b in range(2):
        d = (om[b].float() - of[b, :, L[b] - QS:L[b]].float()).abs().max().item()
        dl = (lm[b] - lf[b, :, L[b] - QS:L[b]]).abs().max().item()
        assert d <= TOL_OUT[torch.bfloat16] and dl <= TOL_LSE, (b, d, dl)
    pf.close()
    pm.close()


def test_paged_prefill_is_invariant_to_pool_permutation():
    a = W.make_paged_prefill("pperm_a", layout="BNSD", B=2, QN=8, KVN=2, D=128, Sq=256,
                             lq=[256, 100], lkv=[1500, 300], block_size=128, seed=350)
    bt = a.block_table.clone()
    NB = a.k.shape[0]
    perm = torch.from_numpy(np.random.default_rng(9).permutation(NB))
    k2 = torch.empty_like(a.k)
    v2 = torch.empty_like(a.v)
    k2[perm] = a.k
    v2[perm] = a.v
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    b = W.make_paged_prefill("pperm_b", layout="BNSD", B=2, QN=8, KVN=2, D=128, Sq=256,
                             lq=[256, 100], lkv=[1500, 300], block_size=128, seed=350)
    b.q, b.k, b.v, b.block_table = a.q, k2, v2, bt2
    to_dev(a)
    to_dev(b)
    pa, pb = fia_plan(a), fia_plan(b)
    oa, la = run(pa)
    ob, lb = run(pb)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    pa.close()
    pb.close()


def test_workload_paged_chunked_prefill_whole_heads():
    # four seeded query heads, every row of every batch
    case = W.paged_chunked_prefill_bf16(device="cuda")
    heads = seeded_subset(case.QN, 4, seed=11)
    rows = head_rows(case, heads)
    say(f"[full] {case.name}: heads {heads}, every row")
    ref_o, ref_l = oracle.attention(case, rows=rows)
    plan = fia_plan(case)
    out, lse = run(plan)
    err, lerr = compare_rows(case, out, lse, rows, ref_o, ref_l)
    say(f"[full] {case.name}: {len(rows)} rows, max out err {err:.3e}, max lse err {lerr:.3e}")
    assert torch.isfinite(out.float()).all()
    plan.close()


def test_workload_paged_mtp_decode_full():
    # every row of the 4-token decode workload
    case = W.paged_mtp_decode_bf16(device="cuda")
    say(f"[full] {case.name}: every row")
    ref_o, ref_l = oracle.attention(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err, lerr = compare(case, out, lse, ref_o, ref_l)
    say(f"[full] {case.name}: max out err {err:.3e}, max lse err {lerr:.3e}")
    plan.close()
