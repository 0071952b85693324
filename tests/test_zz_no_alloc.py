"""GPU checks of the allocation-free phase 2 (fia_run_noalloc): through the
C ABI it must give the same outputs as fia_run / bsa_run with a caller
workspace, bit for bit, on two calls in a row (the second one smaller, so it
runs on the scratch the first one left behind), and refuse plans whose
workspace exceeds the static scratch."""
import pytest
import torch

import workloads as W
from attention_fia_fwd_amd import _abi
from fia_gpu import bsa_plan, fia_plan, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _both(plan):
    """(out, lse) of fia_run / bsa_run with the plan's own workspace, then of
    fia_run_noalloc on the same plan (outputs refilled with NaN between)."""
    plan.out.fill_(float("nan"))
    out_ws, lse_ws = plan.run()
    torch.cuda.synchronize()
    out_ws, lse_ws = out_ws.clone(), None if lse_ws is None else lse_ws.clone()
    plan.out.fill_(float("nan"))
    if plan.lse is not None:
        plan.lse.fill_(float("nan"))
    st = _abi.fia_run_noalloc(plan.plan, _stream())
    assert st == _abi.FIA_OK, _abi.fia_status_string(st)
    torch.cuda.synchronize()
    return out_ws, lse_ws, plan.out, plan.lse


def _check(case, make_plan):
    to_dev(case)
    plan = make_plan(case)
    assert 0 < plan.workspace_size <= _abi.FIA_NOALLOC_MAX_WORKSPACE, plan.workspace_size
    say(f"[noalloc] {case.name}: workspace {plan.workspace_size} B")
    ow, lw, on, ln = _both(plan)
    assert torch.equal(ow, on), f"{case.name}: outputs differ"
    assert lw is None or torch.equal(lw, ln), f"{case.name}: lse differ"
    plan.close()


def test_noalloc_decode_twice_second_smaller():
    # paged GQA decode: the scratch holds the split partial results
    big = W.make_paged_decode("noalloc_decode_big", B=8, QN=32, KVN=8, D=128,
                              lkv=[5000, 17, 900, 3000, 1, 2048, 700, 4096], block_size=128, seed=601)
    _check(big, fia_plan)
    small = W.make_paged_decode("noalloc_decode_small", B=2, QN=8, KVN=2, D=64, lkv=[300, 41],
                                block_size=16, seed=602)
    _check(small, fia_plan)


def test_noalloc_block_sparse_twice_second_smaller():
    # block-sparse: the scratch holds the compacted block lists
    big = W.make_bsa("noalloc_bsa_big", B=1, QN=8, KVN=2, Sq=2000, D=128, X=128, Y=128, p=0.3,
                     seed=603)
    _check(big, bsa_plan)
    small = W.make_bsa("noalloc_bsa_small", B=1, QN=2, KVN=1, Sq=300, D=64, X=128, Y=128, p=0.5,
                       seed=604)
    _check(small, bsa_plan)


def test_noalloc_int8_and_multi_token_decode():
    q8 = W.make_quant_decode("noalloc_int8", B=3, QN=8, KVN=2, D=128, lkv=[1200, 33, 64],
                             kmode=0, vmode=1, block_size=64, seed=605)
    _check(q8, fia_plan)
    mtp = W.make_paged_prefill("noalloc_mtp", layout="BNSD", B=3, QN=8, KVN=2, D=128, Sq=4,
                               lkv=[900, 4, 300], block_size=128, sparse_mode=3, mask_kind="template",
                               seed=606)
    _check(mtp, fia_plan)


def test_noalloc_prefill_needs_no_scratch():
    case = W.make_fia("noalloc_prefill", layout="BSND", dtype=torch.bfloat16, B=2, QN=4, KVN=2,
                      Sq=200, Dqk=128, sparse_mode=3, mask_kind="template", lq=[200, 77],
                      lkv=[200, 77], seed=607)
    to_dev(case)
    plan = fia_plan(case)
    assert plan.workspace_size == 0
    ow, lw, on, ln = _both(plan)
    assert torch.equal(ow, on) and torch.equal(lw, ln)
    plan.close()


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # MLA decode with 128 heads: partials of 128 rows x 512 per piece
    case = W.make_mla_decode("noalloc_mla_big", B=64, QN=128, Sq=1, lkv=[600] * 64, block_size=128,
                             seed=608)
    to_dev(case)
    plan = fia_plan(case)
    assert plan.workspace_size > _abi.FIA_NOALLOC_MAX_WORKSPACE, plan.workspace_size
    plan.out.fill_(float("nan"))
    torch.cuda.synchronize()
    st = _abi.fia_run_noalloc(plan.plan, _stream())
    assert st == _abi.FIA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(plan.out.float()).all()          # nothing was launched
    plan.close()
