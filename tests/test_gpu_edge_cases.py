"""GPU parity at the edges of the parameter ranges: zero and negative
scale_value, the largest GQA ratio (64), 256 query heads, and long
sequences (a 200K-token decode cache, a 20K-row causal prefill), each
against the fp64 oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import (bsa_plan, compare, fia_plan, gather_rows, run, sample_rows, say, to_dev,
                     TOL_LSE, TOL_OUT)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check(case):
    say(f"[edge] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"Sq={case.Sq} Skv={case.Skv} D={case.Dqk} mode={case.sparse_mode} scale={case.scale}")
    ref_out, ref_lse = oracle.attention(case)
    to_dev(case)
    plan = fia_plan(case)
    out, lse = run(plan)
    err = compare(case, out, lse, ref_out, ref_lse)
    plan.close()
    return err


@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_prefill_zero_and_negative_scale(scale):
    # scale 0: every allowed key weighs the same (out = mean of V over the
    # allowed keys, lse = ln |J|); a negative scale flips the scores
    case = W.make_fia(f"prefill_scale_{scale}", layout="BNSD", dtype=torch.bfloat16, B=2, QN=4,
                      KVN=2, Sq=200, Dqk=128, sparse_mode=3, lq=[200, 77], lkv=[200, 77],
                      scale=scale, seed=500)
    check(case)


@pytest.mark.parametrize("scale", [0.0, -0.09])
def test_decode_zero_and_negative_scale(scale):
    case = W.make_paged_decode(f"decode_scale_{scale}", B=3, QN=8, KVN=2, D=128,
                               lkv=[900, 1, 130], block_size=128, scale=scale, seed=501)
    check(case)


def test_bsa_negative_scale():
    case = W.make_bsa("bsa_negscale", layout="BNSD", B=1, QN=2, KVN=1, Sq=384, D=128, X=128,
                      Y=128, p=0.5, scale=-0.07, seed=502)
    say(f"[edge] {case.name}")
    ref_out, ref_lse = oracle.block_sparse(case)
    to_dev(case)
    plan = bsa_plan(case)
    out, lse = run(plan)
    compare(case, out, lse, ref_out, ref_lse)
    plan.close()


def test_prefill_gqa_ratio_64():
    case = W.make_fia("prefill_g64", layout="BSND", dtype=torch.bfloat16, B=2, QN=64, KVN=1,
                      Sq=150, Dqk=128, sparse_mode=3, lq=[150, 33], lkv=[150, 33], seed=503)
    check(case)


def test_decode_gqa_ratio_64():
    # 64 heads of one kv head: four 16-column chunks
    case = W.make_fia("decode_g64", layout="BNSD", dtype=torch.bfloat16, B=2, QN=64, KVN=1,
                      Sq=1, Skv=3000, Dqk=128, lkv=[3000, 17], seed=504)
    check(case)


def test_prefill_256_heads():
    case = W.make_fia("prefill_n256", layout="BNSD", dtype=torch.float16, B=1, QN=256, KVN=256,
                      Sq=70, Dqk=64, sparse_mode=2, mask_kind="template", seed=505)
    check(case)


def test_decode_long_cache():
    # 200K and 70K cached tokens: one (batch, kv head) spans many waves
    case = W.make_fia("decode_long", layout="BSND", dtype=torch.bfloat16, B=2, QN=8, KVN=1,
                      Sq=1, Skv=200000, Dqk=128, lkv=[200000, 70001], seed=506, device="cuda")
    check(case)


def test_prefill_long_sequence_sampled():
    case = W.make_fia("prefill_long", layout="BNSD", dtype=torch.bfloat16, B=1, QN=2, KVN=1,
                      Sq=20000, Dqk=128, sparse_mode=3, lq=[19999], lkv=[19999], seed=507,
                      device="cuda")
    say(f"[edge] {case.name}")
    rows = sample_rows(case, 64, seed=21)
    ref_o, ref_l = oracle.attention(case, rows=rows)
    plan = fia_plan(case)
    out, lse = run(plan)
    go, gl = gather_rows(case, out, lse, rows)
    err = float(np.max(np.abs(go - ref_o)))
    lerr = float(np.max(np.abs(gl - ref_l)))
    say(f"[edge] {case.name}: max out err {err:.3e}, max lse err {lerr:.3e}")
    assert err <= TOL_OUT[case.dtype] and lerr <= TOL_LSE
    # the padding row past the length is 0 / +inf
    assert torch.all(out[0, :, 19999] == 0) and torch.all(torch.isposinf(lse[0, :, 19999]))
    plan.close()
