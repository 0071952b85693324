"""GPU parity of MLA decode (query D 512 + rope 64, one kv head, paged K,
V and K_rope pools) against the fp64 oracle: query layouts, both pool
layouts, block sizes 16 and 128, Q_N from 1 to 128, query S 1..16 with
bottom-right causal masking, kv lengths 0, 1 and ragged, NaN in every pool
row that must not be read, zero and negative scales, and the full-size
workload on whole batches (every head)."""
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import compare, compare_rows, fia_plan, head_rows, run, say, seeded_subset, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


CASES = [
    # name, layout, dtype, QN, S, block_size, pool_layout, lkv, lq
    ("n16_s1_bs16", "BSND", torch.bfloat16, 16, 1, 16, 1, [300, 1, 0, 77], None),
    ("n128_s1_bs128_f16", "BNSD", torch.float16, 128, 1, 128, 0, [1000, 513], None),
    ("n32_s2_bsh", "BSH", torch.bfloat16, 32, 2, 128, 1, [700, 130], None),
    ("n1_s1", "BSND", torch.bfloat16, 1, 1, 16, 0, [95, 33, 16], None),
    ("n2_s4", "BSND", torch.bfloat16, 2, 4, 16, 1, [40, 4, 3], None),
    ("n8_s3_two_waves", "BNSD", torch.bfloat16, 8, 3, 16, 1, [250, 61], None),
    ("n64_s2_eight_waves", "BSND", torch.bfloat16, 64, 2, 128, 0, [900, 2], None),
    ("n128_s4_four_chunks", "BSND", torch.bfloat16, 128, 4, 128, 1, [650, 300], [4, 2]),
    ("n4_s16_f16", "BNSD", torch.float16, 4, 16, 16, 1, [200, 10], None),
    ("n16_s1_long", "BSND", torch.bfloat16, 16, 1, 128, 1, [20000, 3], None),
]


@pytest.mark.parametrize("case_args", CASES, ids=[c[0] for c in CASES])
def test_mla_decode_matches_oracle(case_args):
    name, layout, dtype, QN, S, bs, pl, lkv, lq = case_args
    case = W.make_mla_decode(f"mla_{name}", layout=layout, dtype=dtype, B=len(lkv), QN=QN, Sq=S,
                             lq=lq, lkv=lkv, block_size=bs, pool_layout=pl, seed=1200 + len(name),
                             extra_blocks=2, nan_pool=True)
    say(f"[mla] {case.name} layout={layout} QN={QN} S={S} bs={bs} pool={pl} lkv={lkv} lq={lq} "
        f"dtype={dtype}")
    ref = oracle.attention(case)
    to_dev(case)
    p = fia_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    # a second run of the same plan gives the same bits
    out2, lse2 = run(p)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    p.close()


@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_mla_zero_and_negative_scale(scale):
    case = W.make_mla_decode(f"mla_scale_{scale}", B=2, QN=16, Sq=2, lkv=[300, 40], block_size=16,
                             scale=scale, seed=1230, nan_pool=True)
    say(f"[mla] {case.name}")
    ref = oracle.attention(case)
    to_dev(case)
    p = fia_plan(case)
    compare(case, *run(p), *ref)
    p.close()


@pytest.mark.parametrize("make", [W.mla_decode_bf16, W.mla_decode_shared_kv_bf16],
                         ids=["separate_value", "value_is_key"])
def test_mla_full_size_workload_whole_batches(make):
    # two seeded batches, every one of their 128 query heads
    case = make(device="cuda")
    batches = seeded_subset(case.B, 2, seed=31)
    rows = head_rows(case, range(case.QN), batches=batches)
    say(f"[mla] {case.name}: batches {batches}, every head")
    ref_o, ref_l = oracle.attention(case, rows=rows)
    p = fia_plan(case)
    out, lse = run(p)
    err, lerr = compare_rows(case, out, lse, rows, ref_o, ref_l)
    say(f"[mla] {case.name}: {len(rows)} rows, max out err {err:.3e}, max lse err {lerr:.3e}")
    assert torch.isfinite(out).all()
    p.close()


VK_CASES = [
    # name, layout, QN, S, block_size, pool_layout, lkv
    ("vk_n128_s1", "BSND", 128, 1, 128, 1, [900, 33, 0]),
    ("vk_n16_s4", "BNSD", 16, 4, 16, 0, [400, 5]),
    ("vk_n2_s1", "BSH", 2, 1, 16, 1, [97, 64, 1]),
    ("vk_n64_s2", "BSND", 64, 2, 128, 0, [2100, 130]),
]


@pytest.mark.parametrize("case_args", VK_CASES, ids=[c[0] for c in VK_CASES])
def test_mla_value_is_key(case_args):
    # value passed as the key tensor itself (the latent cache read as both):
    # V comes from the K tiles
    name, layout, QN, S, bs, pl, lkv = case_args
    case = W.make_mla_decode(f"mla_{name}", layout=layout, B=len(lkv), QN=QN, Sq=S, lkv=lkv,
                             block_size=bs, pool_layout=pl, seed=1250 + QN, extra_blocks=2, nan_pool=True)
    case.v = case.k
    say(f"[mla] {case.name} value=key layout={layout} QN={QN} S={S} bs={bs} pool={pl} lkv={lkv}")
    ref = oracle.attention(case)
    to_dev(case)
    case.v = case.k                      # one device tensor for both
    p = fia_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    p.close()


TND_CASES = [
    # name, QN, lq (tokens per batch), lkv, block_size, value = key
    ("tnd_n16_mixed", 16, [1, 3, 16, 2], [300, 50, 1000, 2], 16, False),
    ("tnd_n128_s1", 128, [1, 1, 1], [700, 1, 40], 128, False),
    ("tnd_n8_short_kv", 8, [4, 1], [3, 200], 16, False),
    ("tnd_n32_value_is_key", 32, [2, 5, 1], [600, 130, 0], 128, True),
]


@pytest.mark.parametrize("case_args", TND_CASES, ids=[c[0] for c in TND_CASES])
def test_mla_tnd(case_args):
    # TND query: batch b's lq_b tokens are consecutive rows; kv lengths per
    # batch; rows of a batch with fewer allowed keys than tokens are 0 / +inf
    name, QN, lq, lkv, bs, vk = case_args
    case = W.make_mla_decode(f"mla_{name}", layout="TND", B=len(lq), QN=QN, lq=lq, lkv=lkv,
                             block_size=bs, pool_layout=1, seed=1270 + QN, extra_blocks=2, nan_pool=True)
    if vk:
        case.v = case.k
    say(f"[mla] {case.name} TND QN={QN} lq={lq} lkv={lkv} bs={bs} value=key={vk}")
    ref = oracle.attention(case)
    to_dev(case)
    if vk:
        case.v = case.k
    p = fia_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    p.close()


BAND_CASES = [
    # name, QN, S, block_size, lkv, (pre_tokens, next_tokens), value = key
    ("band_s1_narrow", 16, 1, 16, [900, 40, 5], (100, 0), False),
    ("band_s1_n128", 128, 1, 128, [3000, 700], (1000, 0), False),
    ("band_s4", 16, 4, 16, [600, 3, 70], (50, 0), False),
    ("band_s2_next", 32, 2, 128, [1500, 200], (300, 1), False),
    ("band_s1_zero_window", 8, 1, 16, [400, 17], (0, 0), False),
    ("band_s4_value_is_key", 64, 4, 128, [2500, 90], (700, 0), True),
    ("band_s1_bs64", 128, 1, 64, [2000, 130, 64], (500, 0), False),
]


@pytest.mark.parametrize("case_args", BAND_CASES, ids=[c[0] for c in BAND_CASES])
def test_mla_band(case_args):
    # sparse_mode 4: token t sees keys Lkv - S + t - pre .. Lkv - S + t + next
    # (at query S 1 too); keys below every row's window are not loaded
    name, QN, S, bs, lkv, band, vk = case_args
    case = W.make_mla_decode(f"mla_{name}", B=len(lkv), QN=QN, Sq=S, lkv=lkv, block_size=bs,
                             band=band, seed=1290 + QN + S, extra_blocks=2, nan_pool=True)
    if vk:
        case.v = case.k
    say(f"[mla] {case.name} band={band} QN={QN} S={S} bs={bs} lkv={lkv} value=key={vk}")
    ref = oracle.attention(case)
    to_dev(case)
    if vk:
        case.v = case.k
    p = fia_plan(case)
    out, lse = run(p)
    compare(case, out, lse, *ref)
    p.close()
