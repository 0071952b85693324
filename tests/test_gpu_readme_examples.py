"""The Python examples of README.md, run as written on cuda:0, with their
outputs checked against the fp64 oracle: the causal GQA prefill with ragged
lengths (whole heads, padding rows included) and the MLA decode against a
paged latent cache passed as both key and value (every head of two
batches)."""
import os
import re

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from fia_gpu import compare_rows, head_rows, say, seeded_subset

pytestmark = pytest.mark.gpu

_README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _examples():
    with open(_README, encoding="utf-8") as f:
        return re.findall(r"```python\n(.*?)```", f.read(), flags=re.S)


def _exec(src, prelude=""):
    torch.manual_seed(0)
    ns = {}
    exec(compile(prelude + src, _README, "exec"), ns)
    torch.cuda.synchronize()
    return ns


def test_readme_has_the_two_examples():
    ex = _examples()
    assert len(ex) == 2 and "FiaPlan" in ex[0] and "query_rope" in ex[1]


def test_readme_prefill_example():
    ns = _exec(_examples()[0])
    q, k, v, out, lse = ns["q"], ns["k"], ns["v"], ns["out"], ns["lse"]
    L = np.array([4096, 3000, 1024, 77])
    case = W.FiaCase(name="readme_prefill", layout="BSND", dtype=torch.bfloat16, B=4, QN=32,
                     KVN=8, Sq=4096, Skv=4096, Dqk=128, Dv=128, scale=128 ** -0.5,
                     sparse_mode=3, lq=L, lkv=L, q=q, k=k, v=v)
    heads = seeded_subset(32, 2, seed=41)
    rows = head_rows(case, heads)
    say(f"[readme] prefill: heads {heads}, {len(rows)} rows")
    ref_o, ref_l = oracle.attention(case, rows=rows)
    err, lerr = compare_rows(case, out, lse, rows, ref_o, ref_l)
    say(f"[readme] prefill: max out err {err:.3e}, max lse err {lerr:.3e}")
    # rows past each batch's length: out = 0, lse = +inf
    for b in range(4):
        assert torch.all(out[b, L[b]:] == 0)
        assert torch.all(torch.isposinf(lse[b, :, L[b]:]))


def test_readme_mla_example():
    # the second example continues the first: it runs after the first's imports
    ex = _examples()
    imports = "".join(ln + "\n" for ln in ex[0].splitlines() if ln.startswith("import "))
    ns = _exec(ex[1], prelude=imports)
    ckv, kpe, q, q_pe, table, out = (ns[n] for n in ("ckv", "kpe", "q", "q_pe", "table", "out"))
    case = W.FiaCase(name="readme_mla", layout="BSND", dtype=torch.bfloat16, B=64, QN=128, KVN=1,
                     Sq=1, Skv=64 * 128, Dqk=512, Dv=512, scale=576 ** -0.5, sparse_mode=0,
                     lq=np.ones(64, dtype=np.int64), lkv=np.full(64, 8192), q=q, k=ckv, v=ckv,
                     block_table=table, block_size=128, pool_layout=1, return_lse=False,
                     rope={"query_rope": q_pe, "key_rope": kpe})
    batches = seeded_subset(64, 2, seed=43)
    rows = head_rows(case, range(128), batches=batches)
    say(f"[readme] MLA: batches {batches}, every head")
    ref_o, ref_l = oracle.attention(case, rows=rows)
    err, _ = compare_rows(case, out, None, rows, ref_o, ref_l)
    say(f"[readme] MLA: max out err {err:.3e}")
    assert torch.isfinite(out.float()).all()
