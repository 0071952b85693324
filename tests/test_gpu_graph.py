"""Phase 2 only enqueues kernels (no allocation, no memset, no
synchronization), so a run can be captured in a HIP graph.  Each case runs
eagerly, is captured once, and is replayed several times with eager work
and synchronizations between the replays and the outputs refilled with NaN
before each; every replay must reproduce the eager result bit for bit."""
import pytest
import torch

import workloads as W
from fia_gpu import bsa_plan, fia_plan, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


CASES = {
    "prefill_gqa_causal": lambda: W.make_fia("g_prefill", layout="BSND", B=2, QN=8, KVN=2, Sq=300,
                                             Dqk=128, sparse_mode=3, lq=[300, 77], lkv=[300, 77],
                                             mask_kind="template", seed=1300),
    "paged_decode": lambda: W.make_paged_decode("g_decode", B=3, QN=8, KVN=2, D=128,
                                                lkv=[900, 1, 130], block_size=64, seed=1301),
    "int8_decode": lambda: W.make_quant_decode("g_int8", B=2, QN=8, KVN=2, D=128, lkv=[700, 33],
                                               kmode=0, vmode=1, seed=1302),
    "mla_decode": lambda: W.make_mla_decode("g_mla", B=2, QN=16, Sq=2, lkv=[500, 60], block_size=16,
                                            seed=1303),
    "block_sparse": lambda: W.make_bsa("g_bsa", B=1, QN=4, KVN=2, Sq=400, D=128, X=128, Y=128,
                                       p=0.5, seed=1304),
    "fp8_block_sparse": lambda: W.make_bsa_fp8("g_fp8", B=1, QN=2, KVN=1, Sq=300, D=128, Y=256,
                                               p=0.5, seed=1305),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    case = CASES[name]()
    say(f"[graph] {name}")
    to_dev(case)
    bsa = name in ("block_sparse", "fp8_block_sparse")
    p = bsa_plan(case) if bsa else fia_plan(case)
    out, lse = p.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), (lse.clone() if lse is not None else None)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        p.run()                              # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.run()
    torch.cuda.synchronize()

    x = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        p.out.fill_(float("nan"))
        if p.lse is not None:
            p.lse.fill_(float("nan"))
        x = x * 1.0001 + 1.0                 # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(p.out, ref_out), f"{name}: replay {rep} output differs"
        if ref_lse is not None:
            assert torch.equal(p.lse, ref_lse), f"{name}: replay {rep} lse differs"
    del g
    p.close()
