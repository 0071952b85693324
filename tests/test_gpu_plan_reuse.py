"""Phase 1 keeps its temporaries (and the host image of the schedule tables)
in per-thread buffers that are reused from call to call.  These tests build
plans of every kind interleaved with each other and from several threads at
once, and check that each plan's runs are bitwise identical to those of the
same plan built alone, first in the process; and that independent plans run
at the same time on two streams give the same bits as run alone."""
import threading

import pytest
import torch

import workloads as W
from fia_gpu import bsa_plan, fia_plan, run, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _cases():
    """A prefill with padding rows (zero-fill workgroups), a varlen TND
    prefill, a paged decode, an MLA decode and a block-sparse prefill: every
    planner path, with table images of very different sizes."""
    return [
        ("prefill", W.make_fia("reuse_prefill", layout="BSND", dtype=torch.bfloat16, B=3, QN=8, KVN=2,
                               Sq=700, Dqk=128, sparse_mode=3, lq=[700, 129, 400], lkv=[700, 129, 400],
                               seed=301, mask_kind="template")),
        ("tnd", W.make_fia("reuse_tnd", layout="TND", dtype=torch.bfloat16, B=3, QN=4, KVN=4, Dqk=64,
                           sparse_mode=3, lq=[300, 77, 512], lkv=[300, 77, 512], seed=302,
                           mask_kind="template")),
        ("decode", W.make_paged_decode("reuse_decode", B=5, QN=8, KVN=2, D=128, lkv=[900, 17, 4000, 1, 2500],
                                       block_size=64, seed=303)),
        ("mla", W.make_mla_decode("reuse_mla", B=3, QN=64, Sq=1, lkv=[700, 1500, 90], block_size=64,
                                  seed=304)),
        ("bsa", W.make_bsa("reuse_bsa", layout="BNSD", B=1, QN=4, KVN=2, Sq=1000, D=64, X=128, Y=128,
                           p=0.3, seed=305)),
    ]


def _plan(case):
    return (bsa_plan if hasattr(case, "block_mask") else fia_plan)(case)


def _outputs(plan):
    out, lse = run(plan)
    return out.clone(), (lse.clone() if lse is not None else None)


def _same(a, b):
    assert torch.equal(a[0], b[0])
    if a[1] is not None:
        assert torch.equal(a[1], b[1])


def test_plans_built_interleaved_match_plans_built_alone():
    cases = _cases()
    for _, c in cases:
        to_dev(c)
    ref = {}
    for name, c in cases:
        say(f"[reuse] alone: {name}")
        p = _plan(c)
        ref[name] = _outputs(p)
        p.close()
    # every plan built again after each of the others (the scratch buffers
    # then hold the previous plan's larger or smaller tables), all kept alive
    # together, then run in reverse order
    plans = []
    for rnd in range(2):
        for name, c in (cases if rnd == 0 else cases[::-1]):
            say(f"[reuse] round {rnd}: {name}")
            plans.append((name, _plan(c)))
    for name, p in plans[::-1]:
        _same(_outputs(p), ref[name])
        p.close()


def test_plans_built_on_several_threads_at_once():
    cases = _cases()
    for _, c in cases:
        to_dev(c)
    ref = {}
    for name, c in cases:
        p = _plan(c)
        ref[name] = _outputs(p)
        p.close()
    built, errors = {}, []
    barrier = threading.Barrier(len(cases))

    def build(name, case):
        try:
            torch.cuda.set_device(0)
            barrier.wait()
            for _ in range(3):                     # the last of three plans is kept
                p = _plan(case)
                old = built.get(name)
                built[name] = p
                if old is not None:
                    old.close()
        except Exception as e:                     # reported on the main thread
            errors.append((name, repr(e)))

    say("[reuse] phase 1 on %d threads" % len(cases))
    threads = [threading.Thread(target=build, args=(n, c)) for n, c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for name, p in built.items():
        _same(_outputs(p), ref[name])
        p.close()


def test_plans_run_concurrently_on_two_streams():
    """Independent plans (each with its own workspace) in flight at the same
    time on two streams of default priority: every run equals the plan's run
    alone on the default stream, bitwise.  Outputs are refilled with NaN
    before each round, so each round must write every element."""
    cases = _cases()
    for _, c in cases:
        to_dev(c)
    plans = [(name, _plan(c)) for name, c in cases]
    ref = {}
    for name, p in plans:
        say(f"[streams] alone: {name}")
        ref[name] = _outputs(p)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(4):
        for _, p in plans:
            p.out.fill_(float("nan"))
            if p.lse is not None:
                p.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[streams] round {rnd}: {len(plans)} plans on two streams")
        for i, (_, p) in enumerate(plans[::-1] if rnd % 2 else plans):
            with torch.cuda.stream(streams[i % 2]):
                p.run()
        torch.cuda.synchronize()
        for name, p in plans:
            _same((p.out, p.lse), ref[name])
    for _, p in plans:
        p.close()
