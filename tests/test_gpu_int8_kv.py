"""GPU parity of decode against an int8 KV cache (kv pseudo-quantization):
the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs, each cached value standing for scale * (x + offset) per channel or
per token."""
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import compare, fia_plan, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check(case):
    say(f"[int8] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"S={case.Sq} lkv={list(case.lkv)} D={case.Dqk} kmode={case.quant['key_quant_mode']} "
        f"vmode={case.quant['value_quant_mode']} "
        f"offsets={case.quant['dequant_offset_key'] is not None} mode={case.sparse_mode}")
    ref_out, ref_lse = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err = compare(case, out, lse, ref_out, ref_lse)
    plan.close()
    return err


@pytest.mark.parametrize("kmode, vmode", [(0, 0), (1, 1), (0, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_int8_decode_modes(kmode, vmode, D):
    case = W.make_quant_decode(f"int8_k{kmode}v{vmode}_d{D}", layout="BNSD", B=4, QN=8, KVN=2, D=D,
                               lkv=[1500, 1, 33, 700], kmode=kmode, vmode=vmode,
                               seed=400 + 4 * kmode + 2 * vmode + D)
    check(case)


@pytest.mark.parametrize("layout, G, offsets", [("BSND", 4, False), ("BSH", 1, True), ("BNSD", 16, True)])
def test_int8_decode_layouts_gqa_offsets(layout, G, offsets):
    case = W.make_quant_decode(f"int8_{layout}_g{G}", layout=layout, B=3, QN=2 * G, KVN=2, D=128,
                               lkv=[2000, 17, 0], kmode=0, vmode=1, offsets=offsets, seed=410 + G)
    check(case)


@pytest.mark.parametrize("S, G, mode", [(2, 8, 1), (4, 4, 0)])
def test_int8_multi_token_decode(S, G, mode):
    # query S > 1: the two quant modes are equal
    case = W.make_quant_decode(f"int8_mtp{S}_g{G}", layout="BNSD", B=3, QN=2 * G, KVN=2, D=128,
                               Sq=S, lkv=[900, S, 64], kmode=mode, vmode=mode, sparse_mode=3,
                               seed=420 + S)
    check(case)


def test_int8_decode_negative_scale():
    case = W.make_quant_decode("int8_negscale", layout="BNSD", B=2, QN=4, KVN=1, D=128,
                               lkv=[300, 45], kmode=0, vmode=0, scale=-0.05, seed=430)
    check(case)


PAGED_CASES = [
    # name, layout, QN, KVN, D, block_size, pool_layout, kmode, vmode, lkv
    ("bs32_pl0_k0v0", "BNSD", 8, 2, 128, 32, 0, 0, 0, [1500, 1, 33, 0, 64]),
    ("bs64_pl1_k1v1", "BSND", 16, 2, 128, 64, 1, 1, 1, [3000, 65, 2]),
    ("bs128_pl0_k0v1", "BSH", 4, 4, 64, 128, 0, 0, 1, [700, 128, 129]),
    ("bs256_pl1_k0v0", "BNSD", 32, 8, 128, 256, 1, 0, 0, [5000, 31]),
    ("bs32_pl1_long", "BNSD", 8, 1, 128, 32, 1, 1, 1, [4200, 2049]),
]


@pytest.mark.parametrize("case_args", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_int8_paged_decode(case_args):
    # page attention with an int8 cache (query S 1): pages gathered through
    # the block table in both pool layouts; pieces of more than 64 pages at
    # block 32 exercise the planner's cap on pages per piece
    name, layout, QN, KVN, D, bs, pl, km, vm, lkv = case_args
    case = W.make_quant_decode(f"int8_paged_{name}", layout=layout, B=len(lkv), QN=QN, KVN=KVN, D=D,
                               lkv=lkv, kmode=km, vmode=vm, block_size=bs, pool_layout=pl,
                               extra_blocks=3, seed=440 + bs + 2 * km + vm)
    check(case)


def test_int8_paged_pool_permutation_bitwise():
    # one cache placed in the pool under two different seeded permutations:
    # the split schedule does not depend on the block ids, so the outputs
    # are bitwise identical
    a = W.make_quant_decode("int8_pg_a", layout="BNSD", B=3, QN=8, KVN=2, D=128, lkv=[900, 77, 256],
                            kmode=0, vmode=1, block_size=64, seed=460)
    b = W.make_quant_decode("int8_pg_b", layout="BNSD", B=3, QN=8, KVN=2, D=128, lkv=[900, 77, 256],
                            kmode=0, vmode=1, block_size=64, seed=461)
    # b: the pages of a placed at b's block ids
    bt_a, bt_b = a.block_table.numpy(), b.block_table.numpy()
    kb, vb = torch.zeros_like(a.k), torch.zeros_like(a.v)
    for bb in range(3):
        for c in range(bt_a.shape[1]):
            if bt_a[bb, c] >= 0:
                kb[bt_b[bb, c]] = a.k[bt_a[bb, c]]
                vb[bt_b[bb, c]] = a.v[bt_a[bb, c]]
    b.q, b.k, b.v, b.quant = a.q, kb, vb, dict(a.quant)
    to_dev(a)
    to_dev(b)
    pa, pb = fia_plan(a), fia_plan(b)
    oa, la = run(pa)
    ob, lb = run(pb)
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    pa.close()
    pb.close()


def test_workload_int8_kv_decode_full():
    # every row of the contiguous int8 decode workload
    case = W.int8_kv_decode_bf16(device="cuda")
    say(f"[full] {case.name}: every row")
    ref_o, ref_l = oracle.attention(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err, lerr = compare(case, out, lse, ref_o, ref_l)
    say(f"[full] {case.name}: max out err {err:.3e}, max lse err {lerr:.3e}")
    plan.close()


def test_workload_int8_paged_decode_full():
    # every row of the paged int8 decode workload (the paged GQA decode
    # shape with an int8 pool)
    case = W.int8_paged_decode_bf16(device="cuda")
    say(f"[full] {case.name}: every row")
    ref_o, ref_l = oracle.attention(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err, lerr = compare(case, out, lse, ref_o, ref_l)
    say(f"[full] {case.name}: max out err {err:.3e}, max lse err {lerr:.3e}")
    plan.close()
