"""GPU parity of block-sparse attention with FP8 (E4M3FN) query, key and
value and per-block fp32 dequant scales: the HIP path through the C ABI
against the fp64 oracle on the same seeded inputs (bf16 output, tolerances
of the bf16 path)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import bsa_plan, compare, compare_rows, head_rows, run, say, seeded_subset, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def check(case):
    say(f"[fp8] {case.name} layout={case.layout} B={case.B} QN={case.QN} KVN={case.KVN} "
        f"Sq={case.Sq} Skv={case.Skv} Y={case.Y} lq={case.lq} lkv={case.lkv}")
    ref_out, ref_lse = oracle.block_sparse(case)
    to_dev(case)
    plan = bsa_plan(case)
    out, lse = run(plan)
    assert out.dtype == torch.bfloat16
    err = compare(case, out, lse, ref_out, ref_lse)
    plan.close()
    return err


@pytest.mark.parametrize("Y", [256, 512])
@pytest.mark.parametrize("layout", ["BNSD", "BSND"])
def test_bsa_fp8_blocks_layouts(Y, layout):
    case = W.make_bsa_fp8(f"fp8_{layout}_y{Y}", layout=layout, B=2, QN=4, KVN=2, Sq=700, Skv=1300,
                          D=128, Y=Y, p=0.5, lq=[700, 129], lkv=[1300, 300], seed=600 + Y)
    check(case)


def test_bsa_fp8_all_selected_and_negative_scale():
    case = W.make_bsa_fp8("fp8_ones_negscale", layout="BNSD", B=1, QN=8, KVN=1, Sq=384, D=128,
                          Y=256, mask_kind="ones", scale=-0.08, seed=610)
    check(case)


def test_bsa_fp8_tnd():
    L = np.array([500, 64, 1000])
    # TND: a [T, N, D] layout built from per-sequence BNSD draws
    seqs = [W.make_bsa_fp8("s", layout="BNSD", B=1, QN=4, KVN=2, Sq=int(n), D=128, Y=256, p=0.6,
                           seed=620 + i) for i, n in enumerate(L)]
    q = torch.cat([s.q[0].permute(1, 0, 2) for s in seqs]).contiguous()
    k = torch.cat([s.k[0].permute(1, 0, 2) for s in seqs]).contiguous()
    v = torch.cat([s.v[0].permute(1, 0, 2) for s in seqs]).contiguous()
    nqb, nkb = -(-int(L.max()) // 128), -(-int(L.max()) // 256)

    def padded(key, nb, N):
        out = torch.zeros(3, N, nb, 1, dtype=torch.float32)
        for i, s in enumerate(seqs):
            t = s.fp8[key][0]
            out[i, :, :t.shape[1]] = t
        return out

    m = np.zeros((3, 4, nqb, nkb), dtype=np.uint8)
    for i, s in enumerate(seqs):
        bm = s.block_mask.numpy()[0]
        m[i, :, :bm.shape[1], :bm.shape[2]] = bm
    case = W.BsaCase(name="fp8_tnd", layout="TND", dtype=torch.float8_e4m3fn, B=3, QN=4, KVN=2,
                     Sq=int(L.sum()), Skv=int(L.sum()), D=128, X=128, Y=256,
                     scale=1.0 / np.sqrt(128), lq=L, lkv=L, q=q, k=k, v=v,
                     block_mask=torch.from_numpy(m),
                     fp8={"dequant_scale_query": padded("dequant_scale_query", nqb, 4),
                          "dequant_scale_key": padded("dequant_scale_key", nkb, 2),
                          "dequant_scale_value": padded("dequant_scale_value", nkb, 2)})
    check(case)


def test_workload_fp8_block_sparse_whole_heads():
    # two seeded query heads, every row of each (32768 rows per head)
    case = W.fp8_block_sparse(device="cuda")
    heads = seeded_subset(case.QN, 2, seed=31)
    rows = head_rows(case, heads)
    say(f"[full] {case.name}: heads {heads}, every row")
    ref_o, ref_l = oracle.block_sparse(case, rows=rows)
    plan = bsa_plan(case)
    out, lse = run(plan)
    err, lerr = compare_rows(case, out, lse, rows, ref_o, ref_l)
    say(f"[full] {case.name}: {len(rows)} rows, max out err {err:.3e}, max lse err {lerr:.3e}")
    assert torch.isfinite(out.float()).all()
    plan.close()
