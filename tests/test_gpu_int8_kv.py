"""GPU parity of decode against an int8 KV cache (kv pseudo-quantization):
the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs, each cached value standing for scale * (x + offset) per channel or
per token."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import compare, fia_plan, gather_rows, run, sample_rows, say, to_dev, TOL_LSE, TOL_OUT

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


@pytest.mark.parametrize("kmode, vmode", [(0, 0), (1, 1), (0, 1), (1, 0)])
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


@pytest.mark.parametrize("S, G", [(2, 8), (4, 4)])
def test_int8_multi_token_decode(S, G):
    case = W.make_quant_decode(f"int8_mtp{S}_g{G}", layout="BNSD", B=3, QN=2 * G, KVN=2, D=128,
                               Sq=S, lkv=[900, S, 64], kmode=1, vmode=0, sparse_mode=3,
                               seed=420 + S)
    check(case)


def test_int8_decode_negative_scale():
    case = W.make_quant_decode("int8_negscale", layout="BNSD", B=2, QN=4, KVN=1, D=128,
                               lkv=[300, 45], kmode=0, vmode=0, scale=-0.05, seed=430)
    check(case)


def test_workload_int8_kv_decode_full_sampled():
    case = W.int8_kv_decode_bf16(device="cuda")
    say(f"[full] {case.name}")
    rows = sample_rows(case, 128, seed=13, decode=True)
    ref_o, ref_l = oracle.attention(case, rows=rows)
    plan = fia_plan(case)
    out, lse = run(plan)
    go, gl = gather_rows(case, out, lse, rows)
    err = float(np.max(np.abs(go - ref_o)))
    lerr = float(np.max(np.abs(gl - ref_l)))
    say(f"[full] {case.name}: {len(rows)} rows, max out err {err:.3e}, max lse err {lerr:.3e}")
    assert err <= TOL_OUT[torch.bfloat16] and lerr <= TOL_LSE
    assert torch.isfinite(out.float()).all()
    plan.close()
