"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element, at sizes that span several tiles
and ragged tails, plus the invariants that hold at any size."""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import (bsa_plan, compare, compare_rows, fia_plan, gather_rows, head_rows, run,
                     sample_rows, say, seeded_subset, to_dev, TOL_OUT, TOL_LSE)

pytestmark = pytest.mark.gpu

INT_MAX = W.INT_MAX


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check_fia(case, **over):
    say(f"[fia] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"Sq={case.Sq} Skv={case.Skv} D={case.Dqk}/{case.Dv} mode={case.sparse_mode} "
        f"dtype={case.dtype}")
    ref_out, ref_lse = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case, **over)
    out, lse = run(plan)
    err = compare(case, out, lse, ref_out, ref_lse)
    plan.close()
    return err


# ---------------------------------------------------------------------------
# prefill: every layout, mask mode, dtype and head dim, ragged tails
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["BNSD", "BSND", "BSH"])
@pytest.mark.parametrize("mode", [0, 2, 3, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_prefill_modes_layouts(layout, mode, dtype):
    case = W.make_fia(f"prefill_{layout}_m{mode}", layout=layout, dtype=dtype, B=2, QN=4, KVN=2,
                      Sq=300, Skv=333, Dqk=128, sparse_mode=mode, pre_tokens=77, next_tokens=45,
                      lq=[300, 170], lkv=[333, 101], seed=100 + mode,
                      mask_kind="template" if mode >= 2 else None)
    check_fia(case)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_head_dims_and_gqa(D):
    case = W.make_fia(f"prefill_d{D}", layout="BNSD", dtype=torch.bfloat16, B=3, QN=8, KVN=2,
                      Sq=257, Dqk=D, sparse_mode=3, lq=[257, 1, 130], lkv=[257, 5, 130], seed=110)
    check_fia(case)


@pytest.mark.parametrize("QN,KVN", [(24, 8), (12, 2), (16, 2), (32, 2)])
@pytest.mark.parametrize("mode", [3, 4])
def test_prefill_gqa_head_groups(QN, KVN, mode):
    # G = 3, 6, 8, 16: workgroups pack 1, 2, 4, 4 heads of a GQA group with
    # 128, 64, 32, 32 rows each; lengths cut through those row blocks
    case = W.make_fia(f"prefill_g{QN // KVN}_m{mode}", layout="BSND", dtype=torch.bfloat16, B=2,
                      QN=QN, KVN=KVN, Sq=290, Skv=310, Dqk=128, sparse_mode=mode, pre_tokens=100,
                      next_tokens=20, lq=[290, 97], lkv=[310, 131], mask_kind="template",
                      seed=130 + QN + mode)
    check_fia(case)


def test_prefill_gqa_explicit_mask():
    # the masked instantiation with 4 heads per workgroup
    case = W.make_fia("prefill_g8_mask", layout="BNSD", dtype=torch.float16, B=2, QN=16, KVN=2,
                      Sq=150, Skv=170, Dqk=64, sparse_mode=0, pre_tokens=60, next_tokens=10,
                      lq=[150, 77], lkv=[170, 90], mask_kind="random", seed=141)
    check_fia(case)


def _repeat_runs(case, plan, rows, ref_o, ref_l, runs=3):
    # One plan run several times: the schedule the plan uploaded once is
    # reused, so every run must write every output row again (outputs are
    # refilled with NaN before each run), match the oracle on the sampled
    # rows and reproduce the first run bit for bit.
    first = None
    for rep in range(runs):
        plan.out.fill_(float("nan"))
        if plan.lse is not None:
            plan.lse.fill_(float("nan"))
        out, lse = run(plan)
        assert not torch.isnan(out.float()).any(), f"run {rep}: tiles left unwritten"
        assert lse is None or not torch.isnan(lse).any(), f"run {rep}: lse left unwritten"
        if first is None:
            go, gl = gather_rows(case, out, lse, rows)
            err = float(np.max(np.abs(go - ref_o)))
            lerr = float(np.max(np.abs(gl - ref_l)))
            say(f"[repeat] {case.name}: max out err {err:.3e}, max lse err {lerr:.3e}")
            assert err <= TOL_OUT[case.dtype] and lerr <= TOL_LSE
            first = (out.clone(), None if lse is None else lse.clone())
        else:
            assert torch.equal(out, first[0]), f"run {rep} differs from the first"
            assert lse is None or torch.equal(lse, first[1])


def test_prefill_repeated_runs_of_one_plan():
    # 2 x 8 kv heads x 64 row blocks = 1024 tiles: more than the resident
    # workgroups, so queues run dry and workgroups steal from other XCDs
    case = W.make_fia("prefill_repeat", layout="BSND", dtype=torch.bfloat16, B=2, QN=32, KVN=8,
                      Sq=2048, Dqk=128, sparse_mode=3, lq=[2048, 1500], lkv=[2048, 1500], seed=150)
    say(f"[repeat] {case.name}")
    rows = sample_rows(case, 48, seed=5)
    ref_o, ref_l = oracle.attention(case, rows=rows)
    to_dev(case)
    plan = fia_plan(case)
    _repeat_runs(case, plan, rows, ref_o, ref_l)
    plan.close()


def test_bsa_repeated_runs_of_one_plan():
    case = W.make_bsa("bsa_repeat", layout="BNSD", B=1, QN=16, KVN=4, Sq=8192, D=128, X=128, Y=128,
                      p=0.1, seed=151, device="cuda")
    say(f"[repeat] {case.name}")
    rows = sample_rows(case, 48, seed=6)
    ref_o, ref_l = oracle.block_sparse(case, rows=rows)
    plan = bsa_plan(case)
    _repeat_runs(case, plan, rows, ref_o, ref_l)
    plan.close()


def test_prefill_tnd_192_128():
    L = [200, 1, 64, 129, 511]
    case = W.make_fia("prefill_tnd_192", layout="TND", dtype=torch.bfloat16, B=5, QN=4, KVN=4,
                      Dqk=192, Dv=128, sparse_mode=3, lq=L, lkv=L, seed=111)
    check_fia(case)


def test_prefill_tnd_unequal_lengths_mode3_and_mode0():
    lq, lkv = [100, 30, 257], [180, 30, 300]
    case = W.make_fia("prefill_tnd_unequal", layout="TND", dtype=torch.bfloat16, B=3, QN=4, KVN=2,
                      Dqk=128, sparse_mode=3, lq=lq, lkv=lkv, seed=112)
    check_fia(case)
    case0 = W.make_fia("prefill_tnd_mode0", layout="TND", dtype=torch.bfloat16, B=3, QN=4, KVN=2,
                       Dqk=128, sparse_mode=0, lq=lq, lkv=lkv, seed=113)
    check_fia(case0)


@pytest.mark.parametrize("mode", [0, 1])
def test_prefill_explicit_masks(mode):
    case = W.make_fia(f"prefill_mask_m{mode}", layout="BNSD", dtype=torch.float16, B=2, QN=2,
                      Sq=150, Skv=200, Dqk=64, sparse_mode=mode, pre_tokens=60, next_tokens=10,
                      lq=[150, 77], lkv=[200, 90], mask_kind="random", seed=120 + mode)
    check_fia(case)


def test_prefill_fully_masked_rows_and_padding():
    # mode 3 with Lkv < Lq leaves the first rows without keys; padding rows
    # past Lq hold NaN that must never be read.
    case = W.make_fia("prefill_empty_rows", layout="BSND", dtype=torch.bfloat16, B=2, QN=2, KVN=1,
                      Sq=200, Skv=200, Dqk=128, sparse_mode=3, lq=[200, 150], lkv=[130, 60],
                      seed=121, nan_padding=True)
    check_fia(case)


def test_prefill_empty_kv_batch():
    case = W.make_fia("prefill_empty_kv", layout="BNSD", dtype=torch.bfloat16, B=2, QN=2, Sq=70,
                      Dqk=64, sparse_mode=0, lq=[70, 70], lkv=[70, 0], seed=122)
    check_fia(case)


def test_prefill_without_lse():
    case = W.make_fia("prefill_nolse", layout="BNSD", dtype=torch.bfloat16, B=1, QN=2, Sq=130,
                      Dqk=128, sparse_mode=2, seed=123, return_lse=False)
    ref_out, _ = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    assert lse is None
    compare(case, out, None, ref_out, None)
    plan.close()


def test_prefill_is_deterministic():
    case = to_dev(W.make_fia("prefill_det", layout="BSND", dtype=torch.bfloat16, B=2, QN=8,
                             KVN=2, Sq=513, Dqk=128, sparse_mode=3, lq=[513, 300],
                             lkv=[513, 300], seed=124))
    plan = fia_plan(case)
    o1, l1 = run(plan)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = run(plan)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    plan.close()


# ---------------------------------------------------------------------------
# decode: contiguous and paged KV, both pool layouts, GQA group sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_contiguous(layout, G):
    KVN = 2
    case = W.make_fia(f"decode_{layout}_g{G}", layout=layout, dtype=torch.bfloat16, B=3,
                      QN=KVN * G, KVN=KVN, Sq=1, Skv=1500, Dqk=128, lkv=[1500, 1, 777],
                      seed=130 + G)
    check_fia(case)


@pytest.mark.parametrize("pool_layout", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_paged(pool_layout, D):
    case = W.make_paged_decode(f"decode_paged_p{pool_layout}_d{D}", dtype=torch.bfloat16, B=4,
                               QN=8, KVN=2, D=D, lkv=[3000, 17, 1, 640], block_size=64,
                               pool_layout=pool_layout, seed=140 + pool_layout, extra_blocks=3)
    check_fia(case)


@pytest.mark.parametrize("layout, G, D", [("BNSD", 1, 128), ("BSND", 4, 64), ("BSH", 8, 128)])
def test_decode_atten_mask_contiguous(layout, G, D):
    # query S == 1 with a (B, 1, 1, KV_S) mask, half of the kv tokens masked
    KVN = 2
    case = W.make_fia(f"decode_mask_{layout}_g{G}", layout=layout, dtype=torch.bfloat16, B=3,
                      QN=KVN * G, KVN=KVN, Sq=1, Skv=1500, Dqk=D, lkv=[1500, 3, 777],
                      mask_kind="random", seed=180 + G)
    check_fia(case)


@pytest.mark.parametrize("mask_shape", ["BS", "B1S"])
def test_decode_atten_mask_paged(mask_shape):
    case = W.make_paged_decode(f"decode_mask_paged_{mask_shape}", dtype=torch.float16, B=4, QN=8,
                               KVN=2, D=128, lkv=[3000, 17, 1, 640], block_size=64,
                               pool_layout=1, seed=185, extra_blocks=2, mask_p=0.3,
                               mask_shape=mask_shape)
    check_fia(case)


def test_decode_atten_mask_fully_masked_batch_and_broadcast():
    case = W.make_fia("decode_mask_full", layout="BNSD", dtype=torch.bfloat16, B=3, QN=8, KVN=2,
                      Sq=1, Skv=900, Dqk=128, lkv=[900, 500, 64], seed=187)
    m = (np.random.default_rng(3).random((3, 900)) < 0.2).astype(np.uint8)
    m[1] = 1                                   # batch 1: no key left
    case.atten_mask = torch.from_numpy(m)
    check_fia(case)
    bc = W.make_fia("decode_mask_bcast", layout="BNSD", dtype=torch.bfloat16, B=3, QN=8, KVN=2,
                    Sq=1, Skv=900, Dqk=128, lkv=[900, 500, 64], seed=187)
    bc.atten_mask = torch.from_numpy(m[:1].copy())   # a leading 1 broadcasts
    check_fia(bc)


def test_decode_fp16_gqa32_and_empty_kv():
    case = W.make_paged_decode("decode_fp16_g32", dtype=torch.float16, B=2, QN=32, KVN=1, D=128,
                               lkv=[900, 0], block_size=128, seed=150)
    check_fia(case)


def test_decode_paged_is_invariant_to_pool_permutation():
    a = W.make_paged_decode("perm_a", B=3, QN=8, KVN=2, D=128, lkv=[2000, 700, 64],
                            block_size=128, seed=160)
    # same logical cache in a differently permuted pool
    bt = a.block_table.clone()
    NB = a.k.shape[0]
    perm = torch.from_numpy(np.random.default_rng(7).permutation(NB))
    k2 = torch.empty_like(a.k)
    v2 = torch.empty_like(a.v)
    k2[perm] = a.k
    v2[perm] = a.v
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    b = W.make_paged_decode("perm_b", B=3, QN=8, KVN=2, D=128, lkv=[2000, 700, 64],
                            block_size=128, seed=160)
    b.q, b.k, b.v, b.block_table = a.q, k2, v2, bt2
    to_dev(a)
    to_dev(b)
    pa, pb = fia_plan(a), fia_plan(b)
    oa, la = run(pa)
    ob, lb = run(pb)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    pa.close()
    pb.close()


def test_decode_equals_last_prefill_row_on_gpu():
    L = [600, 129]
    pre = W.make_fia("dec_vs_prefill", layout="BNSD", dtype=torch.bfloat16, B=2, QN=8, KVN=2,
                     Sq=600, Dqk=128, sparse_mode=3, lq=L, lkv=L, seed=170)
    dec = W.make_fia("dec_vs_prefill_d", layout="BNSD", dtype=torch.bfloat16, B=2, QN=8, KVN=2,
                     Sq=1, Skv=600, Dqk=128, lkv=L, seed=0)
    dec.q = torch.stack([pre.q[b, :, L[b] - 1:L[b]] for b in range(2)]).contiguous()
    dec.k, dec.v = pre.k, pre.v
    to_dev(pre)
    to_dev(dec)
    pp, pd = fia_plan(pre), fia_plan(dec)
    op, lp = run(pp)
    od, ld = run(pd)
    for b in range(2):
        d = (op[b, :, L[b] - 1].float() - od[b, :, 0].float()).abs().max().item()
        assert d <= 2 * TOL_OUT[torch.bfloat16]
        assert (lp[b, :, L[b] - 1, 0] - ld[b, :, 0, 0]).abs().max().item() <= 2 * TOL_LSE
    pp.close()
    pd.close()


# ---------------------------------------------------------------------------
# block-sparse
# ---------------------------------------------------------------------------

def check_bsa(case):
    say(f"[bsa] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"Sq={case.Sq} Skv={case.Skv} D={case.D} X={case.X} Y={case.Y}")
    ref_out, ref_lse = oracle.block_sparse(case)
    lq = case.lq if case.lq is not None else np.full(case.B, case.Sq)
    lkv = case.lkv if case.lkv is not None else np.full(case.B, case.Skv)
    ridx, rcnt = oracle.bsa_compact(case.block_mask.cpu().numpy(), lq, lkv, case.X, case.Y)
    to_dev(case)
    plan = bsa_plan(case)
    out, lse = run(plan)
    cnt, idx, nqb, nkb = plan.schedule()
    assert np.array_equal(cnt.cpu().numpy(), rcnt.reshape(-1)), "compacted counts differ"
    assert np.array_equal(idx.cpu().numpy(), ridx.reshape(-1, nkb)), "compacted lists differ"
    err = compare(case, out, lse, ref_out, ref_lse)
    plan.close()
    return err


@pytest.mark.parametrize("X,Y", [(128, 128), (64, 128), (200, 256)])
def test_bsa_block_shapes(X, Y):
    case = W.make_bsa(f"bsa_{X}x{Y}", layout="BNSD", B=2, QN=4, KVN=2, Sq=700, Skv=900, D=128,
                      X=X, Y=Y, p=0.3, lq=[700, 333], lkv=[900, 257], seed=180)
    check_bsa(case)


@pytest.mark.parametrize("layout", ["BSND", "TND"])
def test_bsa_layouts(layout):
    kw = dict(lq=[300, 129], lkv=[260, 400]) if layout == "TND" else dict(Sq=300, Skv=400)
    case = W.make_bsa(f"bsa_{layout}", layout=layout, B=2, QN=4, KVN=1, D=64, X=128, Y=128,
                      p=0.5, seed=181, dtype=torch.float16, **kw)
    check_bsa(case)


def test_bsa_all_ones_equals_dense_on_gpu():
    case = W.make_bsa("bsa_ones", layout="BNSD", B=1, QN=4, KVN=2, Sq=384, D=128, X=128, Y=128,
                      mask_kind="ones", seed=182)
    check_bsa(case)
    dense = W.make_fia("bsa_ones_dense", layout="BNSD", dtype=torch.bfloat16, B=1, QN=4, KVN=2,
                       Sq=384, Dqk=128, sparse_mode=0, scale=case.scale, seed=0)
    dense.q, dense.k, dense.v = case.q, case.k, case.v
    pb, pd = bsa_plan(case), fia_plan(dense)
    ob, lb = run(pb)
    od, ld = run(pd)
    assert (ob.float() - od.float()).abs().max().item() <= TOL_OUT[torch.bfloat16]
    assert (lb - ld).abs().max().item() <= TOL_LSE
    pb.close()
    pd.close()


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark
# times, against oracle rows sampled one by one
# ---------------------------------------------------------------------------

def test_workload_c1_full():
    check_fia(W.c1_dense_causal_fp16())


def test_workload_c1_mode1_explicit_causal_mask():
    # the smallest workload with sparse_mode 1 and an explicit 128 x 128
    # causal mask (nonzero above the diagonal): the oracle's result, and the
    # mode-3 run's result
    case = W.c1_dense_causal_fp16()
    case.sparse_mode = 1
    case.atten_mask = torch.triu(torch.ones(128, 128, dtype=torch.uint8), diagonal=1)
    check_fia(case)
    p = fia_plan(case)
    out1, lse1 = run(p)
    p.close()
    c3 = to_dev(W.c1_dense_causal_fp16())
    p = fia_plan(c3)
    out3, lse3 = run(p)
    p.close()
    assert (out1.float() - out3.float()).abs().max().item() <= 1e-3
    assert (lse1 - lse3).abs().max().item() <= 1e-5


def _full_whole(case):
    """Every row of the output (padding rows included: out 0, lse +inf)
    against the oracle, element by element."""
    say(f"[full] {case.name}: oracle over every row")
    t0 = time.perf_counter()
    ref_o, ref_l = oracle.attention(case)
    say(f"[full] {case.name}: oracle {time.perf_counter() - t0:.1f} s")
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err, lerr = compare(case, out, lse, ref_o, ref_l)
    say(f"[full] {case.name}: every row, max out err {err:.3e}, max lse err {lerr:.3e}")
    plan.close()


def test_workload_c2_full():
    _full_whole(W.c2_gqa_causal_bf16(device="cuda"))


def test_workload_c3_full():
    case = W.c3_paged_decode_bf16(device="cuda")
    say(f"[full] {case.name}")
    ref_o, ref_l = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err, lerr = compare(case, out, lse, ref_o, ref_l)
    say(f"[full] {case.name}: max out err {err:.3e}, max lse err {lerr:.3e}")
    plan.close()


def test_workload_c4_full():
    _full_whole(W.c4_varlen_tnd_bf16(device="cuda"))


def test_workload_c5_whole_heads():
    # two seeded query heads, every row of each (32768 rows per head)
    case = W.c5_block_sparse_bf16(device="cuda")
    heads = seeded_subset(case.QN, 2, seed=3)
    say(f"[full] {case.name}: heads {heads}, every row")
    rows = head_rows(case, heads)
    ref_o, ref_l = oracle.block_sparse(case, rows=rows)
    ridx, rcnt = oracle.bsa_compact(case.block_mask.cpu().numpy(), np.full(1, case.Sq),
                                    np.full(1, case.Skv), case.X, case.Y)
    plan = bsa_plan(case)
    out, lse = run(plan)
    cnt, idx, nqb, nkb = plan.schedule()
    assert np.array_equal(cnt.cpu().numpy(), rcnt.reshape(-1))
    assert np.array_equal(idx.cpu().numpy(), ridx.reshape(-1, nkb))
    err, lerr = compare_rows(case, out, lse, rows, ref_o, ref_l)
    say(f"[full] {case.name}: {len(rows)} rows, max out err {err:.3e}, max lse err {lerr:.3e}")
    assert torch.isfinite(out.float()).all()
    plan.close()
